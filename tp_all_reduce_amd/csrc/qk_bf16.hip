// QK-norm kernels with bf16 input and output.
#include "kernels.h"

namespace arrms {

QkLaunch pick_qk_bf16(int W, int ppl, bool loop, bool aligned) {
    return pick_qk<Bf16>(W, ppl, loop, aligned);
}

}  // namespace arrms
