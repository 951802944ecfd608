// Reduce + RMSNorm kernels with bf16 input and output, no FP8 epilogue.
#include "kernels.h"

namespace arrms {

Variant pick_rms_bf16(int W, int mode, bool res, bool round) {
    return pick_rms<Bf16, false>(W, mode, res, round);
}

}  // namespace arrms
