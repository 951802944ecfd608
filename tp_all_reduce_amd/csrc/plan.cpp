// Plans, dispatch predicate and argument validation of libarrms.  Host-only
// C++: no HIP calls, so every path here runs (and is tested) without a GPU.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <new>

#include "arrms_host.h"

namespace arrms {

namespace {
thread_local char g_error[512] = "";

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int round_up(int x, int m) { return (x + m - 1) / m * m; }

int next_pow2(int x) {
    int p = 1;
    while (p < x) p <<= 1;
    return p;
}
}  // namespace

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_error[0] = '\0'; }

// Row-resident: one workgroup per token row, one 16-byte pack per lane, the
// whole row held in registers across up to 16 wavefronts.
Shape row_shape(int64_t H) {
    int packs = int(H / kPackElems);
    return Shape{round_up(packs, 64), 1};
}

// Split: the same one-pack-per-lane tiling up to 1024 packs (8192 elements),
// four packs per lane on at most 512 lanes beyond (strided by the workgroup
// size, so every load instruction of a wavefront covers 1 KiB of contiguous
// memory); a persistent grid of workgroups loops over rows.
Shape split_shape(int64_t H) {
    int packs = int(H / kPackElems);
    int ppl = packs <= kMaxBlock ? 1 : kMaxPpl;
    int block = round_up((packs + ppl - 1) / ppl, 64);
    return Shape{block, ppl};
}

// QK-norm with every shard on whole wavefronts: the fewest packs per lane
// (1, 2 or 4) for which W * lanes_for(q + kv packs) fits one workgroup;
// {0, 0} when none does.  Exception, from measurement: four or more shards
// that would fill all 1024 lanes with one pack per lane take two (sixteen
// wavefronts ran 2-10 % slower than eight there; with fewer shards, or fewer
// wavefronts, halving the wavefronts ran as fast or slower).
Shape qk_aligned_shape(int W, int q_size, int kv_size) {
    const int per_shard = (q_size + kv_size) / kPackElems;
    for (int ppl = 1; ppl <= kMaxQkPpl; ppl *= 2) {
        const int lanes = round_up((per_shard + ppl - 1) / ppl, 64);
        if (int64_t(W) * lanes > kMaxBlock) continue;
        if (ppl == 1 && W >= 4 && W * lanes == kMaxBlock) continue;
        return Shape{W * lanes, ppl};
    }
    return Shape{0, 0};
}

Shape qk_shape(int W, int q_size, int kv_size) {
    int packs = W * (q_size + kv_size) / kPackElems;
    int ppl = next_pow2((packs + kMaxBlock - 1) / kMaxBlock);
    int block = round_up((packs + ppl - 1) / ppl, 64);
    return Shape{block, ppl};
}

static int check_plan(const ar_rms_plan_s *plan) {
    if (plan == nullptr) return fail(ARRMS_EINVAL, "plan is NULL");
    return ARRMS_OK;
}

// With T == 0 the [T, H] buffers are empty and may have no address at all.
static int check_partials(const ar_rms_plan_s *plan, const void *const *ptrs, const char *what) {
    if (ptrs == nullptr) return fail(ARRMS_EINVAL, "%s pointer array is NULL", what);
    for (int r = 0; r < plan->W; ++r) {
        if (ptrs[r] == nullptr) {
            if (plan->T == 0) continue;
            return fail(ARRMS_EINVAL, "%s[%d] is NULL", what, r);
        }
        if (!aligned(ptrs[r], 16))
            return fail(ARRMS_EINVAL, "%s[%d] is not 16-byte aligned", what, r);
    }
    return ARRMS_OK;
}

static int check_eps(float eps) {
    if (!std::isfinite(eps) || eps < 0.0f)
        return fail(ARRMS_EINVAL, "eps must be finite and >= 0 (got %g)", double(eps));
    return ARRMS_OK;
}

int check_rms_args(const ar_rms_plan_s *plan, const void *const *partials,
                   const void *residual, const void *weight, float eps,
                   const void *norm_out, bool norm_required, const void *residual_out) {
    int rc;
    if ((rc = check_plan(plan))) return rc;
    if ((rc = check_partials(plan, partials, "partials"))) return rc;
    if (residual != nullptr && !aligned(residual, 16))
        return fail(ARRMS_EINVAL, "residual is not 16-byte aligned");
    if (weight == nullptr) return fail(ARRMS_EINVAL, "weight is NULL");
    if (!aligned(weight, 16)) return fail(ARRMS_EINVAL, "weight is not 16-byte aligned");
    if (norm_required && norm_out == nullptr && plan->T != 0)
        return fail(ARRMS_EINVAL, "norm_out is NULL");
    if (norm_out != nullptr && !aligned(norm_out, 16))
        return fail(ARRMS_EINVAL, "norm_out is not 16-byte aligned");
    if (residual_out != nullptr && !aligned(residual_out, 16))
        return fail(ARRMS_EINVAL, "residual_out is not 16-byte aligned");
    if ((rc = check_eps(eps))) return rc;
    return ARRMS_OK;
}

int check_quant_args(const ar_rms_plan_s *plan, int group_size, const void *q_out,
                     const void *scales) {
    if (group_size < 8 || group_size > 512 || (group_size & (group_size - 1)) != 0)
        return fail(ARRMS_ENOTSUP, "group_size %d is not a power of two in [8, 512]",
                    group_size);
    if (plan->H % group_size != 0)
        return fail(ARRMS_ENOTSUP, "group_size %d does not divide H=%lld", group_size,
                    (long long)plan->H);
    if (q_out == nullptr && plan->T != 0) return fail(ARRMS_EINVAL, "q_out is NULL");
    if (!aligned(q_out, 8)) return fail(ARRMS_EINVAL, "q_out is not 8-byte aligned");
    if (scales == nullptr && plan->T != 0) return fail(ARRMS_EINVAL, "scales is NULL");
    if (!aligned(scales, 4)) return fail(ARRMS_EINVAL, "scales is not 4-byte aligned");
    return ARRMS_OK;
}

int check_qk_args(const ar_rms_plan_s *plan, const void *const *qkv, int q_size, int kv_size,
                  const void *q_weight, const void *k_weight, float eps, const void *q_out,
                  const void *k_out) {
    int rc;
    if ((rc = check_plan(plan))) return rc;
    if (q_size <= 0 || kv_size <= 0)
        return fail(ARRMS_EINVAL, "q_size and kv_size must be positive (got %d, %d)", q_size,
                    kv_size);
    if (plan->W > kMaxQkW)
        return fail(ARRMS_ENOTSUP, "QK-norm takes at most %d shards (got W=%d)", kMaxQkW,
                    plan->W);
    // 32 lanes x one 16-byte pack of 8 elements
    const int align = 32 * kPackElems;
    if (q_size % align != 0 || kv_size % align != 0)
        return fail(ARRMS_ENOTSUP, "q_size %d and kv_size %d must be multiples of %d", q_size,
                    kv_size, align);
    if (int64_t(q_size) + 2 * int64_t(kv_size) != plan->H)
        return fail(ARRMS_ENOTSUP, "q_size + 2*kv_size = %lld does not match the plan's H=%lld",
                    (long long)(int64_t(q_size) + 2 * int64_t(kv_size)), (long long)plan->H);
    if (int64_t(plan->W) * (q_size + kv_size) / kPackElems > int64_t(kMaxBlock) * kMaxQkPpl)
        return fail(ARRMS_ENOTSUP, "W*(q_size+kv_size) = %lld exceeds %lld elements",
                    (long long)plan->W * (q_size + kv_size),
                    (long long)kMaxBlock * kMaxQkPpl * kPackElems);
    if ((rc = check_partials(plan, qkv, "qkv"))) return rc;
    if (q_weight == nullptr || k_weight == nullptr)
        return fail(ARRMS_EINVAL, "q_weight and k_weight must not be NULL");
    if (!aligned(q_weight, 16) || !aligned(k_weight, 16))
        return fail(ARRMS_EINVAL, "q_weight and k_weight must be 16-byte aligned");
    if ((q_out == nullptr || k_out == nullptr) && plan->T != 0)
        return fail(ARRMS_EINVAL, "q_out and k_out must not be NULL");
    if (!aligned(q_out, 16) || !aligned(k_out, 16))
        return fail(ARRMS_EINVAL, "q_out and k_out must be 16-byte aligned");
    return check_eps(eps);
}

}  // namespace arrms

using namespace arrms;

extern "C" int ar_rms_one_stage(int W, int64_t T, int64_t H, int dtype, int fully_connected) {
    // Token cap first, then format, then 16-byte packs (at most 1024 per row),
    // then the per-topology byte caps of the one-stage all-reduce.
    if (W < 1 || T < 0 || H <= 0) return 0;
    if (T > kMaxRowTokens) return 0;
    if (dtype != ARRMS_BF16 && dtype != ARRMS_FP16) return 0;
    const int64_t elem = 2;
    const int64_t pack = 16 / elem;
    if (H % pack != 0 || H / pack > 1024) return 0;
    if (W == 2) return 1;
    if (!fully_connected) return 0;
    const int64_t bytes = T * H * elem;
    if (W <= 4) return bytes < 256 * 1024 ? 1 : 0;
    if (W <= 8) return bytes < 128 * 1024 ? 1 : 0;
    return 0;
}

extern "C" int ar_rms_plan(int W, int64_t T, int64_t H, int dtype, uint32_t flags,
                           ar_rms_plan_t *out) {
    clear_error();
    if (out == nullptr) return fail(ARRMS_EINVAL, "out is NULL");
    *out = nullptr;
    if (W < 1) return fail(ARRMS_EINVAL, "W must be >= 1 (got %d)", W);
    if (T < 0) return fail(ARRMS_EINVAL, "T must be >= 0 (got %lld)", (long long)T);
    if (H <= 0) return fail(ARRMS_EINVAL, "H must be > 0 (got %lld)", (long long)H);
    if (dtype != ARRMS_BF16 && dtype != ARRMS_FP16)
        return fail(ARRMS_EINVAL, "unknown dtype %d", dtype);
    const uint32_t known = ARRMS_FORCE_ROW | ARRMS_FORCE_SPLIT | ARRMS_ROUND_REDUCED;
    if (flags & ~known) return fail(ARRMS_EINVAL, "unknown flag bits 0x%x", flags & ~known);
    if ((flags & ARRMS_FORCE_ROW) && (flags & ARRMS_FORCE_SPLIT))
        return fail(ARRMS_EINVAL, "FORCE_ROW and FORCE_SPLIT are exclusive");
    if (W > kMaxW) return fail(ARRMS_ENOTSUP, "W=%d exceeds %d partial buffers", W, kMaxW);
    if (W > kMaxPrefetchW && H / kPackElems > kMaxBlock)
        return fail(ARRMS_ENOTSUP, "W=%d > %d needs H <= %d (got H=%lld)", W, kMaxPrefetchW,
                    kMaxBlock * kPackElems, (long long)H);
    if (H % kPackElems != 0)
        return fail(ARRMS_ENOTSUP, "H=%lld is not a multiple of %d (16-byte packs)",
                    (long long)H, kPackElems);
    if (H > kMaxH) return fail(ARRMS_ENOTSUP, "H=%lld exceeds %lld", (long long)H,
                               (long long)kMaxH);
    int kernel;
    if (flags & ARRMS_FORCE_ROW) {
        if (W > kMaxPrefetchW)
            return fail(ARRMS_ENOTSUP, "FORCE_ROW needs W <= %d (got W=%d)", kMaxPrefetchW, W);
        if (T > kMaxRowTokens || H / kPackElems > 1024)
            return fail(ARRMS_ENOTSUP,
                        "FORCE_ROW needs T <= 80 and H/8 <= 1024 (got T=%lld, H=%lld)",
                        (long long)T, (long long)H);
        kernel = ARRMS_KERNEL_ROW;
    } else if (flags & ARRMS_FORCE_SPLIT) {
        kernel = ARRMS_KERNEL_SPLIT;
    } else {
        kernel = ar_rms_one_stage(W, T, H, dtype, 1) ? ARRMS_KERNEL_ROW : ARRMS_KERNEL_SPLIT;
    }
    auto *p = new (std::nothrow) ar_rms_plan_s;
    if (p == nullptr) return fail(ARRMS_ENOMEM, "out of host memory");
    Shape s = kernel == ARRMS_KERNEL_ROW ? row_shape(H) : split_shape(H);
    *p = ar_rms_plan_s{W, T, H, dtype, flags, kernel, s.block, s.ppl};
    *out = p;
    return ARRMS_OK;
}

extern "C" void ar_rms_plan_destroy(ar_rms_plan_t plan) { delete plan; }

extern "C" int ar_rms_plan_kernel(const ar_rms_plan_s *plan) {
    if (plan == nullptr) return fail(ARRMS_EINVAL, "plan is NULL");
    return plan->kernel;
}

extern "C" const char *ar_rms_last_error(void) { return g_error; }
