/*
 * libarrms -- fused W-way reduce + residual add + RMSNorm for MI355X (gfx950).
 *
 * The tensor-parallel layer epilogue "all-reduce the partial sums, add the
 * residual, RMS-normalise" (vLLM PR #54787 page, "Motivation" and the
 * fused_allreduce_gemma_rms_norm / _rocm_aiter_fused_allreduce_rmsnorm_impl
 * excerpts under "Key source excerpts"), computed on one GPU: the W per-rank
 * partial-sum buffers are already resident in this GPU's memory and the kernel
 * reduces them itself.  Variants: a per-group FP8 (OCP E4M3FN) quantisation of
 * the normalised output (same page, "Implementation breakdown" item 2: the
 * per-group-quant ops, with and without the 16-bit norm output), and the
 * MiniMax QK-norm whose per-token statistics are reduced across the W shards
 * (vLLM PR #44849 page, "Implementation breakdown" and the
 * _minimax_qk_norm_fusion excerpt).
 *
 * Conventions shared by every entry point
 *  - Pointers named "device" are HIP device pointers owned by the caller; the
 *    library never allocates, frees, synchronises or reads device memory on the
 *    host, so every *_run call can be captured into a HIP graph.
 *  - Activations are row-major, contiguous [T, H] of the plan's 16-bit format;
 *    T is the token count numel / H over all leading dimensions (vLLM PR #49673
 *    page, "Implementation breakdown" item 1).  Device pointers to 16-bit data
 *    must be 16-byte aligned (every lane moves 16-byte packs of 8 elements).
 *  - Every call returns ARRMS_OK or a negative status and never returns OK
 *    without having queued the work that writes all requested outputs; on an
 *    error nothing is launched and no output is touched.  This rules out the
 *    failure the PR #54787 page warns about under "Risks and impact" item 1: an
 *    older fused kernel that returned without writing its outputs.
 *    ar_rms_last_error() gives a message for the last non-OK status of the
 *    calling thread.
 *  - Work is queued on `stream` (a hipStream_t; NULL is the null stream) and is
 *    asynchronous; calls that overlap on their outputs race.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef ARRMS_H
#define ARRMS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
    ARRMS_OK = 0,
    ARRMS_EINVAL = -1,  /* malformed argument: null/misaligned pointer, bad size, bad eps */
    ARRMS_ENOTSUP = -2, /* well-formed but outside what the kernels cover: the caller
                           falls back to the unfused path, as the callers on the pages
                           do (PR #54787 page, "Key source excerpts": the all_reduce +
                           norm branch of fused_allreduce_gemma_rms_norm; PR #44849
                           page, "Key source excerpts": the final fallback of
                           _minimax_qk_norm_fusion) */
    ARRMS_EHIP = -3,    /* the HIP runtime refused the launch */
    ARRMS_ENOMEM = -4   /* host memory for a plan could not be allocated */
};

/* 16-bit activation formats (the fused op admits only these; PR #54787 page,
 * "Key source excerpts": dtype bf16 or fp16). */
enum { ARRMS_BF16 = 0, ARRMS_FP16 = 1 };

/* Plan flags. */
enum {
    ARRMS_FORCE_ROW = 1u << 0,     /* row-resident kernel; needs T <= 80 and H/8 <= 1024 */
    ARRMS_FORCE_SPLIT = 1u << 1,   /* split (multi-row, bandwidth) kernel; always valid */
    /* Round the W-way fp32 sum to the 16-bit format before the residual is added,
     * as the unfused path does, whose all-reduce returns a 16-bit tensor (PR #54787
     * page, "Key source excerpts": the fallback of fused_allreduce_gemma_rms_norm).
     * Without it the sum stays fp32 until residual_out is rounded once. */
    ARRMS_ROUND_REDUCED = 1u << 2
};

/* Kernel chosen by a plan (ar_rms_plan_kernel). */
enum { ARRMS_KERNEL_ROW = 0, ARRMS_KERNEL_SPLIT = 1 };

/* Opaque, immutable, host-only plan; safe to share between threads. */
typedef struct ar_rms_plan_s ar_rms_plan_s;
typedef ar_rms_plan_s *ar_rms_plan_t;

/*
 * The one-stage window predicate (PR #54787 page, "Implementation breakdown"
 * item 1 and the use_1stage_fused_ar_rms excerpt): returns 1 when T <= 80, the
 * format is bf16/fp16, H is a whole number of 16-byte packs and at most 1024 of
 * them, and then either W == 2, or the group is fully connected and the input's
 * T*H*2 bytes are below 256 KiB (W <= 4) or 128 KiB (W <= 8); returns 0
 * otherwise (including W > 8, negative sizes and unknown formats).  Depends
 * only on its arguments (capture-static).
 */
int ar_rms_one_stage(int W, int64_t T, int64_t H, int dtype, int fully_connected);

/*
 * Builds a plan for W partial buffers of [T, H] in format `dtype`.  The kernel
 * is the row-resident one when ar_rms_one_stage(W, T, H, dtype, 1) holds (an
 * MI355X xGMI group is fully connected) and the split one otherwise, unless a
 * FORCE flag says which.  W may exceed the pages' eight ranks (up to 16, for
 * rows of at most 8192 elements); such plans always use the split kernel.
 * Errors: EINVAL for out == NULL, W < 1, T < 0, H <= 0, unknown dtype, unknown
 * flag bits or both FORCE flags; ENOTSUP for W > 16, W > 8 with H > 8192,
 * H % 8 != 0, H > 16384, or FORCE_ROW with W > 8, T > 80 or H/8 > 1024;
 * ENOMEM.  On success *out owns a host allocation released by
 * ar_rms_plan_destroy.
 */
int ar_rms_plan(int W, int64_t T, int64_t H, int dtype, uint32_t flags, ar_rms_plan_t *out);

/* Releases a plan (NULL is ignored).  Work already queued with it is unaffected. */
void ar_rms_plan_destroy(ar_rms_plan_t plan);

/* ARRMS_KERNEL_ROW or ARRMS_KERNEL_SPLIT; ARRMS_EINVAL for NULL. */
int ar_rms_plan_kernel(const ar_rms_plan_s *plan);

/*
 * Fused reduce + residual add + RMSNorm (PR #54787 page, "Key source excerpts":
 * _rocm_aiter_fused_allreduce_rmsnorm_impl and its fake, which returns outputs
 * shaped like the input and the residual).  For every token row t, element h:
 *   y          = (((P_0 + P_1) + ...) + P_{W-1}) + R         in fp32, this order
 *                (with ARRMS_ROUND_REDUCED the sum of the P_r is rounded to the
 *                16-bit format before R is added)
 *   residual_out = round_to_dtype(y)                          (nearest-even)
 *   norm_out   = round_to_dtype(y * rsqrt(sum_h y^2 / H + eps) * w_eff)
 * with w_eff = w (gemma == 0) or 1 + w (gemma != 0, Gemma RMSNorm; PR #54787
 * page, "Key source excerpts": gemma_norm=True, weight bias 1.0).
 *   partials      host array of W device pointers, each [T, H] (stand-ins for the
 *                 W ranks' buffers; separate allocations are fine)
 *   residual      device [T, H], or NULL: no residual term
 *   weight        device [H]
 *   eps           finite, >= 0
 *   norm_out      device [T, H]
 *   residual_out  device [T, H], or NULL (dead residual output); may equal
 *                 `residual` (in place); no other overlap is allowed
 *   stream        hipStream_t
 * T == 0 returns OK and launches nothing; the [T, H] pointers may then be NULL
 * (empty tensors).  Rows whose fp32 sum of squares
 * overflows (|y| around 1e19 and above) give 0 or NaN outputs.
 */
int ar_rms_run(const ar_rms_plan_s *plan, const void *const *partials, const void *residual,
               const void *weight, float eps, int gemma, void *norm_out, void *residual_out,
               void *stream);

/*
 * ar_rms_run followed by per-group FP8 quantisation of the normalised row
 * (PR #54787 page, "Implementation breakdown" item 2: the per-group-quant op and
 * the one that also returns the 16-bit norm).  For each group g of `group_size`
 * consecutive elements of row t, with x the fp32 normalised value:
 *   scales[t, g] = max_g |x| / 448                          (fp32)
 *   q_out[t, h]  = E4M3FN(x / scales[t, g]), nearest-even, saturating; 0 when
 *                  the scale is 0
 *   group_size    power of two, 8..512, dividing H (else ENOTSUP)
 *   norm_out      device [T, H] 16-bit, or NULL (codes only)
 *   q_out         device [T, H] uint8, 8-byte aligned
 *   scales        device [T, H / group_size] fp32, 4-byte aligned
 * Other arguments as in ar_rms_run.
 */
int ar_rms_quant_run(const ar_rms_plan_s *plan, const void *const *partials,
                     const void *residual, const void *weight, float eps, int gemma,
                     int group_size, void *norm_out, uint8_t *q_out, float *scales,
                     void *residual_out, void *stream);

/*
 * QK-norm across W tensor-parallel shards (PR #44849 page, "Implementation
 * breakdown" items 3-4 and the custom_fused_qknorm_ar call).  The plan's H is
 * the shard row length q_size + 2 * kv_size; shard r's row t is [q | k | v].
 * For every token t:
 *   rq = rsqrt(sum_r sum_j q_r[t,j]^2 / (W * q_size) + eps)
 *   rk = rsqrt(sum_r sum_j k_r[t,j]^2 / (W * kv_size) + eps)
 *   q_out[r, t, j] = round(q_r[t,j] * rq * q_weight[r * q_size + j])
 *   k_out[r, t, j] = round(k_r[t,j] * rk * k_weight[r * kv_size + j])
 * i.e. RMSNorm of the q (k) heads of all shards concatenated.  v is not read.
 *   qkv        host array of W device pointers, each [T, q_size + 2*kv_size]
 *   q_weight   device [W * q_size];  k_weight  device [W * kv_size]
 *   q_out      device [W, T, q_size];  k_out  device [W, T, kv_size]
 * EINVAL if q_size or kv_size is not positive; ENOTSUP unless both are
 * multiples of 256 (32 lanes of 16-byte packs: the alignment the fused QK
 * kernel requires, PR #44849 page, "Implementation breakdown" item 3) with
 * q_size + 2 * kv_size == H and W * (q_size + kv_size) <= 32768, and unless
 * W <= 8; the plan's FORCE flags do not apply.
 */
int ar_qknorm_run(const ar_rms_plan_s *plan, const void *const *qkv, int q_size, int kv_size,
                  const void *q_weight, const void *k_weight, float eps, void *q_out,
                  void *k_out, void *stream);

/* Message for the calling thread's last non-OK status ("" if none yet).  The
 * pointer stays valid until the thread's next libarrms call. */
const char *ar_rms_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ARRMS_H */
