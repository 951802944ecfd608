// Reduce + RMSNorm kernels with bf16 input and output and the FP8 E4M3FN
// per-group quant epilogue.
#include "kernels.h"

namespace arrms {

Variant pick_rms_bf16_fp8(int W, int mode, bool res, bool round) {
    return pick_rms<Bf16, true>(W, mode, res, round);
}

}  // namespace arrms
