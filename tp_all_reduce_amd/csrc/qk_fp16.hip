// QK-norm kernels with fp16 input and output.
#include "kernels.h"

namespace arrms {

QkLaunch pick_qk_fp16(int W, int ppl, bool loop, bool aligned) {
    return pick_qk<Fp16>(W, ppl, loop, aligned);
}

}  // namespace arrms
