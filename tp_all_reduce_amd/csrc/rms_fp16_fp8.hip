// Reduce + RMSNorm kernels with fp16 input and output and the FP8 E4M3FN
// per-group quant epilogue.
#include "kernels.h"

namespace arrms {

Variant pick_rms_fp16_fp8(int W, int mode, bool res, bool round) {
    return pick_rms<Fp16, true>(W, mode, res, round);
}

}  // namespace arrms
