// Reduce + RMSNorm kernels with fp16 input and output, no FP8 epilogue.
#include "kernels.h"

namespace arrms {

Variant pick_rms_fp16(int W, int mode, bool res, bool round) {
    return pick_rms<Fp16, false>(W, mode, res, round);
}

}  // namespace arrms
