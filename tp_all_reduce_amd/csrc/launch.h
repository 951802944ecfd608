// Launch interface between the kernel units and the run unit of libarrms:
// the parameter blocks the launchers take, the kernel modes, and the variant
// pickers that each kernel unit defines for its slice of the instantiations
// (reduce + RMSNorm for one I/O format with or without the FP8 epilogue, or
// QK-norm for one I/O format).  The kernel units compile in parallel; the run
// unit holds no device code.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "arrms_host.h"

namespace arrms {

// ------------------------------------------------------- reduce + RMSNorm
struct RmsParams {
    const uint8_t *partials[kMaxW];
    const uint8_t *residual;      // NULL: no residual term
    const uint8_t *weight;
    uint8_t *norm_out;            // NULL allowed in the quant variant
    uint8_t *residual_out;        // NULL: dead residual output
    uint8_t *q_out;               // quant variant: [T, H] codes
    float *scales;                // quant variant: [T, H / group]
    int64_t T;
    int32_t H;
    int32_t packs;                // H / 8
    float eps;
    int32_t options;              // kGemma
    int32_t group_lanes;          // group_size / 8
    int32_t groups;               // H / group_size
    int32_t grid;                 // workgroups (the launch's gridDim.x)
};

// Lanes of a workgroup that covers `packs` 16-byte packs with `ppl` packs per
// lane, in whole wavefronts.  The kernels derive their width from it (reading
// blockDim goes through the dispatch packet in memory) and the launchers check
// that the launch agrees.
__host__ __device__ constexpr int lanes_for(int packs, int ppl) {
    return ((packs + ppl - 1) / ppl + 63) / 64 * 64;
}

// Option bits of a reduce+norm call.
constexpr int32_t kGemma = 1;         // weight applied as 1 + w (Gemma RMSNorm)

// Kernel modes.  kRow: one row per workgroup, straight-line code.  kSplit:
// persistent workgroups looping over rows, the next row's loads issued one row
// ahead.  kSplitWide: persistent, loads at the top of each row, for shapes that
// leave no room in registers for a second row: four packs per lane (rows
// longer than 8192 elements), or one pack per lane with more than eight
// partials.  kSplitLean: the kSplitWide body with one pack per lane for four to
// eight partials without the FP8 epilogue; it needs few enough registers for
// two workgroups per CU, which beats the row-ahead loads when each workgroup
// would get only a few rows.  kSplitLeanFew: the same body with the store
// policy for at most two rows per workgroup (norm_out without device scope).
enum Mode { kRow = 0, kSplit = 1, kSplitWide = 2, kSplitLean = 3, kSplitLeanFew = 4 };

// ------------------------------------------------------------- QK-norm
struct QkParams {
    // the W shard pointers as named fields: lanes pick theirs by selects, and
    // an array here would be indexed per lane and placed in scratch memory
    const uint8_t *x0, *x1, *x2, *x3, *x4, *x5, *x6, *x7;
    const uint8_t *q_weight;
    const uint8_t *k_weight;
    uint8_t *q_out;
    uint8_t *k_out;
    int64_t T;
    int32_t q_packs;              // q_size / 8
    int32_t kv_packs;             // kv_size / 8
    float eps;
    int32_t grid;                 // workgroups (the launch's gridDim.x)
};

// ------------------------------------------------------------- launchers
// A launcher checks that the block matches its kernel and enqueues it.
using RmsLaunch = hipError_t (*)(const RmsParams &, unsigned, unsigned, hipStream_t);
using QkLaunch = hipError_t (*)(const QkParams &, unsigned, unsigned, hipStream_t);

// A kernel variant: its launcher and its symbol (for the occupancy query).
struct Variant {
    RmsLaunch launch;
    const void *symbol;
};

// Reduce + RMSNorm variant for W partials, mode (a Mode above), a residual
// term or none, and the reduced sum rounded to the I/O format or not;
// {nullptr, nullptr} when no such kernel is built.  One function per I/O format
// (bf16, fp16) and epilogue (none, FP8 group quant).
Variant pick_rms_bf16(int W, int mode, bool res, bool round);
Variant pick_rms_bf16_fp8(int W, int mode, bool res, bool round);
Variant pick_rms_fp16(int W, int mode, bool res, bool round);
Variant pick_rms_fp16_fp8(int W, int mode, bool res, bool round);

// QK-norm launcher for W shards, `ppl` packs per lane, looping over tokens or
// not, shard-aligned lane layout or packed; nullptr when none is built.
QkLaunch pick_qk_bf16(int W, int ppl, bool loop, bool aligned);
QkLaunch pick_qk_fp16(int W, int ppl, bool loop, bool aligned);

}  // namespace arrms
