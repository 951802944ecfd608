// Run entry points of libarrms: argument checks (plan.cpp), the choice of
// kernel body and grid, and the launch.  The kernels themselves are built in
// the kernel units (rms_*.hip, qk_*.hip), which this unit reaches through the
// variant pickers; it holds no device code.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <vector>

#include "arrms_host.h"
#include "launch.h"

namespace arrms {
namespace {

// The reduce + RMSNorm variant, from the kernel unit of its I/O format and
// epilogue.
Variant pick_rms(int dtype, int W, int mode, bool quant, bool res, bool round) {
    if (dtype == ARRMS_BF16)
        return quant ? pick_rms_bf16_fp8(W, mode, res, round) : pick_rms_bf16(W, mode, res, round);
    return quant ? pick_rms_fp16_fp8(W, mode, res, round) : pick_rms_fp16(W, mode, res, round);
}

// Workgroups of the split kernel that the device holds at once (CUs times
// resident workgroups per CU for this kernel and block size); the persistent
// grid is min(T, this).  Queried once per (device, kernel, block) and cached.
int resident_grid(const void *symbol, int block) {
    struct Entry {
        int device;
        const void *symbol;
        int block;
        int grid;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (const Entry &e : cache)
            if (e.device == dev && e.symbol == symbol && e.block == block) return e.grid;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, symbol, block, 0) != hipSuccess)
        return -1;
    const int grid = cus * (per_cu > 0 ? per_cu : 1);
    std::lock_guard<std::mutex> lock(mu);
    cache.push_back(Entry{dev, symbol, block, grid});
    return grid;
}

int run_rms(const ar_rms_plan_s *plan, const void *const *partials, const void *residual,
            const void *weight, float eps, int gemma, void *norm_out, void *residual_out,
            bool quant, int group_size, uint8_t *q_out, float *scales, void *stream) {
    if (plan->T == 0) return ARRMS_OK;
    RmsParams p{};
    for (int r = 0; r < plan->W; ++r) p.partials[r] = static_cast<const uint8_t *>(partials[r]);
    p.residual = static_cast<const uint8_t *>(residual);
    p.weight = static_cast<const uint8_t *>(weight);
    p.norm_out = static_cast<uint8_t *>(norm_out);
    p.residual_out = static_cast<uint8_t *>(residual_out);
    p.q_out = q_out;
    p.scales = scales;
    p.T = plan->T;
    p.H = int32_t(plan->H);
    p.packs = int32_t(plan->H / kPackElems);
    p.eps = eps;
    p.options = gemma ? kGemma : 0;
    p.group_lanes = quant ? group_size / kPackElems : 1;
    p.groups = quant ? int32_t(plan->H / group_size) : 0;
    // The split plan launches min(T, resident workgroups); when every row gets
    // its own workgroup the straight-line row body is used (the loop costs
    // latency and has nothing to overlap).
    const bool split = plan->kernel == ARRMS_KERNEL_SPLIT;
    int mode = !split ? kRow
                      : (plan->ppl == 1 && plan->W <= kMaxPrefetchW ? kSplit : kSplitWide);
    const bool res = residual != nullptr;
    const bool round = (plan->flags & ARRMS_ROUND_REDUCED) != 0;
    Variant v = pick_rms(plan->dtype, plan->W, mode, quant, res, round);
    if (v.launch == nullptr)
        return fail(ARRMS_ENOTSUP, "no kernel for W=%d, %d packs per lane", plan->W, plan->ppl);
    int64_t grid = plan->T;
    if (split) {
        const int resident = resident_grid(v.symbol, plan->block);
        if (resident <= 0) return fail(ARRMS_EHIP, "device occupancy query failed");
        // At most eight rows per workgroup: without the FP8 epilogue, four to
        // eight partials run faster on twice the workgroups per CU without the
        // row-ahead loads, where the device holds that many (measured 2-4 %
        // faster at 512 to 2048 rows; with more rows, with the FP8 epilogue or
        // with fewer partials the row-ahead body is as fast or faster).
        Variant lean{nullptr, nullptr};
        if (mode == kSplit && grid > resident && grid <= 8 * int64_t(resident))
            lean = pick_rms(plan->dtype, plan->W, kSplitLean, quant, res, round);
        const int lean_resident = lean.launch ? resident_grid(lean.symbol, plan->block) : 0;
        if (lean.launch && lean_resident >= 2 * resident) {
            v = lean;
            grid = grid < lean_resident ? grid : lean_resident;
            // With at most two rows per workgroup a workgroup's stores gather at
            // the end of the call, and norm_out stored at device scope measured
            // 2-3 % slower there (eight partials, 512 and 1024 rows): those
            // plans take the body whose norm_out stores are only non-temporal.
            if (plan->T <= 2 * grid) {
                const Variant few =
                    pick_rms(plan->dtype, plan->W, kSplitLeanFew, quant, res, round);
                if (few.launch) v = few;
            }
        } else if (grid > resident) {
            grid = resident;
        } else if (mode == kSplit) {
            mode = kRow;
            v = pick_rms(plan->dtype, plan->W, mode, quant, res, round);
        }
    }
    hipError_t e = v.launch(p, unsigned(grid), unsigned(plan->block), static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(ARRMS_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ARRMS_OK;
}

}  // namespace
}  // namespace arrms

using namespace arrms;

extern "C" int ar_rms_run(const ar_rms_plan_s *plan, const void *const *partials,
                          const void *residual, const void *weight, float eps, int gemma,
                          void *norm_out, void *residual_out, void *stream) {
    clear_error();
    int rc = check_rms_args(plan, partials, residual, weight, eps, norm_out, true, residual_out);
    if (rc) return rc;
    return run_rms(plan, partials, residual, weight, eps, gemma, norm_out, residual_out, false, 0,
                   nullptr, nullptr, stream);
}

extern "C" int ar_rms_quant_run(const ar_rms_plan_s *plan, const void *const *partials,
                                const void *residual, const void *weight, float eps, int gemma,
                                int group_size, void *norm_out, uint8_t *q_out, float *scales,
                                void *residual_out, void *stream) {
    clear_error();
    int rc = check_rms_args(plan, partials, residual, weight, eps, norm_out, false, residual_out);
    if (rc) return rc;
    rc = check_quant_args(plan, group_size, q_out, scales);
    if (rc) return rc;
    return run_rms(plan, partials, residual, weight, eps, gemma, norm_out, residual_out, true,
                   group_size, q_out, scales, stream);
}

extern "C" int ar_qknorm_run(const ar_rms_plan_s *plan, const void *const *qkv, int q_size,
                             int kv_size, const void *q_weight, const void *k_weight, float eps,
                             void *q_out, void *k_out, void *stream) {
    clear_error();
    int rc = check_qk_args(plan, qkv, q_size, kv_size, q_weight, k_weight, eps, q_out, k_out);
    if (rc) return rc;
    if (plan->T == 0) return ARRMS_OK;
    QkParams p{};
    const uint8_t *const *xs = reinterpret_cast<const uint8_t *const *>(qkv);
    const uint8_t *first = xs[0];
    p.x0 = first;
    p.x1 = plan->W > 1 ? xs[1] : first;
    p.x2 = plan->W > 2 ? xs[2] : first;
    p.x3 = plan->W > 3 ? xs[3] : first;
    p.x4 = plan->W > 4 ? xs[4] : first;
    p.x5 = plan->W > 5 ? xs[5] : first;
    p.x6 = plan->W > 6 ? xs[6] : first;
    p.x7 = plan->W > 7 ? xs[7] : first;
    p.q_weight = static_cast<const uint8_t *>(q_weight);
    p.k_weight = static_cast<const uint8_t *>(k_weight);
    p.q_out = static_cast<uint8_t *>(q_out);
    p.k_out = static_cast<uint8_t *>(k_out);
    p.T = plan->T;
    p.q_packs = q_size / kPackElems;
    p.kv_packs = kv_size / kPackElems;
    p.eps = eps;
    // shards on whole wavefronts when that fits, else packs back to back
    Shape s = qk_aligned_shape(plan->W, q_size, kv_size);
    const bool aligned = s.block != 0;
    if (!aligned) s = qk_shape(plan->W, q_size, kv_size);
    // one workgroup per token; beyond 65536 tokens workgroups loop over tokens
    const int64_t max_grid = 65536;
    const bool loop = plan->T > max_grid;
    const int64_t grid = loop ? max_grid : plan->T;
    QkLaunch fn = plan->dtype == ARRMS_BF16 ? pick_qk_bf16(plan->W, s.ppl, loop, aligned)
                                            : pick_qk_fp16(plan->W, s.ppl, loop, aligned);
    if (fn == nullptr) return fail(ARRMS_ENOTSUP, "no QK kernel for %d packs per lane", s.ppl);
    hipError_t e = fn(p, unsigned(grid), unsigned(s.block), static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(ARRMS_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ARRMS_OK;
}
