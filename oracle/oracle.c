/*
 * Reference oracle for the fused "W-way reduce + residual add + RMSNorm" layer
 * epilogue and its FP8 per-group-quant and QK-norm variants.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct CPU
 * definition that the GPU library is checked against.  Only the tests, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no code,
 * header, table or helper with the GPU library, and the GPU library never calls it.
 *
 * Sources (vLLM pull-request summary pages on prhub.com.cn):
 *   [54787]  PR #54787 page "ROCm 接入 AITER 融合 allreduce+RMSNorm 快路径"
 *            (ROCm AITER fused allreduce+RMSNorm fast path)
 *   [44849]  PR #44849 page "[ROCm][MiniMax-M2] Dispatch fused QK-norm + AllReduce via AITER"
 *   [50802]  PR #50802 page (dead-residual add-RMSNorm fusion, grouped-FP8 test)
 *   [49673]  PR #49673 page "[ROCM] Fix AITER Fused AllReduce RMSNorm for Transformers Backend"
 *
 * What is computed.  The fused op must give the numbers of the unfused composition
 * "all-reduce the W partial sums, add the residual, RMS-normalise" ([54787],
 * "Motivation": the fallback keeps its numerics; "Key source excerpts":
 * fused_allreduce_gemma_rms_norm falls back to tensor_model_parallel_all_reduce
 * followed by the norm).  So this oracle is that plain definition, with these
 * readings where the pages leave a step open:
 *   - the W partials are summed in fp32, rank 0 first, rank W-1 last, and the
 *     residual is added last, still in fp32, with no intermediate rounding to the
 *     16-bit input format;
 *   - residual_out is that fp32 sum rounded once (round-to-nearest-even) to the
 *     input format;
 *   - the norm works on the unrounded fp32 sum; the sum of squares, mean, rsqrt,
 *     weight product are carried in fp64 and rounded once to the output format;
 *   - Gemma RMSNorm scales by (1 + w) instead of w ([54787], "Key source excerpts":
 *     gemma_norm=True, weight bias 1.0);
 *   - FP8 codes are OCP E4M3FN (bias 7, max 448, NaN = S.1111.111, no infinities),
 *     scale = amax / 448 per group of G consecutive elements along the row; the code
 *     decision is made in fp32 from the normalised value rounded to fp32;
 *   - QK-norm: per token, one sum of squares over the q columns of all W shards and
 *     one over the k columns; q and k of every shard are scaled by their own
 *     rsqrt and by the global weight column that shard owns ([44849],
 *     "Implementation breakdown" and "Key source excerpts": custom_fused_qknorm_ar).
 *
 * All 16-bit and 8-bit formats are decoded and encoded from their definitions
 * (sign, biased exponent, fraction), not from any conversion routine, so that the
 * library's conversions can be checked against them.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no fast-math: every
 * float operation is IEEE binary32, every double operation IEEE binary64).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* Number formats                                                            */
/* ------------------------------------------------------------------------- */

/* Format ids.  0 and 1 are the two 16-bit activation formats the fused op admits
 * ([54787], "Key source excerpts": dtype must be bf16 or fp16); 2 is fp32, which
 * only the dispatch predicate sees (and rejects); 3 is the FP8 output format. */
enum { ORC_BF16 = 0, ORC_FP16 = 1, ORC_FP32 = 2, ORC_E4M3 = 3 };

typedef struct {
    int mant_bits;   /* stored fraction bits                       */
    int exp_bits;    /* exponent field width                       */
    int bias;        /* exponent bias                              */
    int emin;        /* exponent of the smallest normal            */
    double maxval;   /* largest finite magnitude                   */
    int has_inf;     /* all-ones exponent encodes inf/NaN (IEEE)   */
} fmt_t;

static fmt_t fmt_of(int f)
{
    fmt_t r;
    switch (f) {
    case ORC_BF16: /* bfloat16: 1-8-7, the top half of IEEE binary32 */
        r.mant_bits = 7; r.exp_bits = 8; r.bias = 127; r.emin = -126;
        r.maxval = ldexp(255.0, 120); r.has_inf = 1; break;        /* (2-2^-7)*2^127 */
    case ORC_FP16: /* IEEE binary16: 1-5-10 */
        r.mant_bits = 10; r.exp_bits = 5; r.bias = 15; r.emin = -14;
        r.maxval = 65504.0; r.has_inf = 1; break;
    default:       /* OCP FP8 E4M3FN: 1-4-3, no inf, only S.1111.111 is NaN */
        r.mant_bits = 3; r.exp_bits = 4; r.bias = 7; r.emin = -6;
        r.maxval = 448.0; r.has_inf = 0; break;
    }
    return r;
}

/* Value of a bit pattern, straight from the format definition. */
double oracle_decode(int f, uint32_t bits)
{
    fmt_t F = fmt_of(f);
    int total = 1 + F.exp_bits + F.mant_bits;
    uint32_t sign = (bits >> (total - 1)) & 1u;
    uint32_t e = (bits >> F.mant_bits) & ((1u << F.exp_bits) - 1u);
    uint32_t m = bits & ((1u << F.mant_bits) - 1u);
    uint32_t emax_field = (1u << F.exp_bits) - 1u;
    double v;
    if (F.has_inf && e == emax_field) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (!F.has_inf && e == emax_field && m == (1u << F.mant_bits) - 1u) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)m, F.emin - F.mant_bits);                     /* subnormal */
    } else {
        v = ldexp(1.0 + ldexp((double)m, -F.mant_bits), (int)e - F.bias); /* normal */
    }
    return sign ? -v : v;
}

/* Round x to the nearest value of format f, ties to the even significand.
 * Overflow: IEEE formats go to infinity when the rounded magnitude exceeds the
 * largest finite value; E4M3FN saturates to +-448 (the OCP "satfinite" mode). */
double oracle_round(int f, double x)
{
    fmt_t F = fmt_of(f);
    if (isnan(x)) return NAN;
    if (isinf(x)) return F.has_inf ? x : copysign(F.maxval, x);
    double a = fabs(x);
    if (a == 0.0) return x;
    int e2;
    frexp(a, &e2);               /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;              /* exponent of the leading bit */
    if (E < F.emin) E = F.emin;  /* subnormal range: fixed quantum */
    double quantum = ldexp(1.0, E - F.mant_bits);
    double r = a / quantum;      /* exact: division by a power of two */
    double n = floor(r);
    double frac = r - n;
    if (frac > 0.5 || (frac == 0.5 && fmod(n, 2.0) == 1.0)) n += 1.0;
    double v = n * quantum;
    if (v > F.maxval) v = F.has_inf ? INFINITY : F.maxval;
    return copysign(v, x);
}

/* Bit pattern of a value that is exactly representable in format f (or +-inf,
 * NaN).  Built field by field from the definition. */
uint32_t oracle_bits(int f, double v)
{
    fmt_t F = fmt_of(f);
    int total = 1 + F.exp_bits + F.mant_bits;
    uint32_t emax_field = (1u << F.exp_bits) - 1u;
    uint32_t sign = signbit(v) ? 1u : 0u;
    uint32_t e, m;
    double a = fabs(v);
    if (isnan(v)) {
        /* canonical quiet NaN: all-ones exponent, top fraction bit (IEEE) or
         * all-ones fraction (E4M3FN) */
        sign = 0;
        e = emax_field;
        m = F.has_inf ? (1u << (F.mant_bits - 1)) : ((1u << F.mant_bits) - 1u);
    } else if (isinf(a)) {
        e = emax_field; m = 0;
    } else if (a < ldexp(1.0, F.emin)) {
        e = 0;
        m = (uint32_t)(a / ldexp(1.0, F.emin - F.mant_bits));
    } else {
        int e2;
        frexp(a, &e2);
        int E = e2 - 1;
        e = (uint32_t)(E + F.bias);
        m = (uint32_t)((a / ldexp(1.0, E) - 1.0) * ldexp(1.0, F.mant_bits));
    }
    return (sign << (total - 1)) | (e << F.mant_bits) | m;
}

uint32_t oracle_encode(int f, double x) { return oracle_bits(f, oracle_round(f, x)); }

/* ------------------------------------------------------------------------- */
/* Dispatch predicate                                                        */
/* ------------------------------------------------------------------------- */

/* Whether the one-stage fused kernel handles an input of `numel` elements with
 * rows of `hidden` elements, element format f, on a tensor-parallel group of W
 * ranks.  Restates the predicate use_1stage_fused_ar_rms ([54787],
 * "Implementation breakdown" item 1 and "Key source excerpts"):
 *   tokens = numel / hidden (all leading dims; [49673], "Implementation
 *   breakdown" item 1) must be at most 80; the format must be bf16 or fp16; a row
 *   must split into 16-byte packs, at most 1024 of them; two ranks always pass;
 *   otherwise the group must be fully connected and the whole input must stay
 *   below 256 KiB (up to 4 ranks) or 128 KiB (up to 8 ranks); more ranks fail. */
int oracle_one_stage(int W, int64_t numel, int64_t hidden, int f, int fully_connected)
{
    if (hidden <= 0) return 0;
    if (numel / hidden > 80) return 0;
    if (f != ORC_BF16 && f != ORC_FP16) return 0;
    int64_t elem = 2;                        /* both admitted formats are 16-bit */
    int64_t pack = 16 / elem;
    if (hidden % pack != 0 || hidden / pack > 1024) return 0;
    if (W == 2) return 1;
    if (!fully_connected) return 0;
    int64_t total_bytes = numel * elem;
    if (W <= 4) return total_bytes < 256 * 1024;
    if (W <= 8) return total_bytes < 128 * 1024;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Reduce + residual add + RMSNorm                                            */
/* ------------------------------------------------------------------------- */

/* Fills, for every token row t:
 *   sum[h]          = fl32(...fl32(fl32(P_0 + P_1) + P_2)... + P_{W-1})     (fp32)
 *   acc[h]          = fl32(sum[h] + R)      or, with round_reduced,
 *                     fl32(round(sum[h]) + R)
 *   residual_out    = round(acc)
 *   rstd            = 1 / sqrt(sum_h acc[h]^2 / H + eps)                     (fp64)
 *   exact[t,h]      = acc[h] * rstd * (gemma ? 1 + w[h] : w[h])               (fp64)
 *   norm_out        = round(exact)
 * round_reduced reproduces the unfused path, whose all-reduce returns the sum as
 * a 16-bit tensor before the residual is added and the row normalised ([54787],
 * "Key source excerpts": the fallback of fused_allreduce_gemma_rms_norm).
 * `partials` is a host array of W pointers to [T,H] bit patterns; residual may be
 * NULL (no residual term, no residual_out); residual_out and exact may be NULL.
 * Returns 0, or -1 on bad arguments. */
int oracle_ar_rms_ex(int W, int64_t T, int64_t H, int f,
                     const uint16_t *const *partials, const uint16_t *residual,
                     const uint16_t *weight, float eps, int gemma, int round_reduced,
                     uint16_t *norm_out, uint16_t *residual_out, double *exact)
{
    if (W < 1 || T < 0 || H <= 0 || (f != ORC_BF16 && f != ORC_FP16)) return -1;
    float *acc = malloc((size_t)H * sizeof *acc);
    if (!acc) return -1;
    for (int64_t t = 0; t < T; ++t) {
        int64_t row = t * H;
        for (int64_t h = 0; h < H; ++h) {
            float s = (float)oracle_decode(f, partials[0][row + h]);
            for (int r = 1; r < W; ++r)
                s = s + (float)oracle_decode(f, partials[r][row + h]);
            if (round_reduced) s = (float)oracle_round(f, (double)s);
            if (residual) s = s + (float)oracle_decode(f, residual[row + h]);
            acc[h] = s;
            if (residual_out) residual_out[row + h] = (uint16_t)oracle_encode(f, (double)s);
        }
        double ss = 0.0;
        for (int64_t h = 0; h < H; ++h) ss += (double)acc[h] * (double)acc[h];
        double rstd = 1.0 / sqrt(ss / (double)H + (double)eps);
        for (int64_t h = 0; h < H; ++h) {
            double w = oracle_decode(f, weight[h]);
            double w_eff = gemma ? 1.0 + w : w;
            double y = (double)acc[h] * rstd * w_eff;
            if (exact) exact[row + h] = y;
            norm_out[row + h] = (uint16_t)oracle_encode(f, y);
        }
    }
    free(acc);
    return 0;
}

int oracle_ar_rms(int W, int64_t T, int64_t H, int f,
                  const uint16_t *const *partials, const uint16_t *residual,
                  const uint16_t *weight, float eps, int gemma,
                  uint16_t *norm_out, uint16_t *residual_out, double *exact)
{
    return oracle_ar_rms_ex(W, T, H, f, partials, residual, weight, eps, gemma, 0, norm_out,
                            residual_out, exact);
}

/* As oracle_ar_rms, then per-group FP8 quantisation of the normalised row
 * ([54787], "Implementation breakdown" item 2: the per-group-quant variants;
 * [50802], "Key source excerpts": group quant of the RMSNorm output).
 * For each group g of `group` consecutive elements of row t:
 *   amax        = max |exact|                         (fp64)
 *   scale       = fl32(amax / 448)
 *   code[h]     = E4M3FN_RNE_SAT( fl32( fl32(exact[h]) / scale ) ),  0 if scale == 0
 *   scales[t,g] = scale
 * norm_out may be NULL (codes only). */
int oracle_ar_rms_quant_ex(int W, int64_t T, int64_t H, int f,
                           const uint16_t *const *partials, const uint16_t *residual,
                           const uint16_t *weight, float eps, int gemma, int round_reduced,
                           int64_t group, uint16_t *norm_out, uint8_t *q_out, float *scales,
                           uint16_t *residual_out, double *exact)
{
    if (W < 1 || W > 64 || H <= 0 || group <= 0 || H % group != 0) return -1;
    double *row_exact = malloc((size_t)H * sizeof *row_exact);
    uint16_t *row_norm = malloc((size_t)H * sizeof *row_norm);
    if (!row_exact || !row_norm) { free(row_exact); free(row_norm); return -1; }
    int rc = 0;
    for (int64_t t = 0; t < T && rc == 0; ++t) {
        const uint16_t *prow[64];
        for (int r = 0; r < W; ++r) prow[r] = partials[r] + t * H;
        rc = oracle_ar_rms_ex(W, 1, H, f, prow, residual ? residual + t * H : NULL,
                              weight, eps, gemma, round_reduced, row_norm,
                              residual_out ? residual_out + t * H : NULL, row_exact);
        if (rc) break;
        if (norm_out) memcpy(norm_out + t * H, row_norm, (size_t)H * sizeof *row_norm);
        if (exact) memcpy(exact + t * H, row_exact, (size_t)H * sizeof *row_exact);
        for (int64_t g = 0; g < H / group; ++g) {
            double amax = 0.0;
            for (int64_t j = 0; j < group; ++j) {
                double a = fabs(row_exact[g * group + j]);
                if (a > amax) amax = a;
            }
            float scale = (float)(amax / 448.0);
            scales[t * (H / group) + g] = scale;
            for (int64_t j = 0; j < group; ++j) {
                int64_t h = g * group + j;
                uint8_t code = 0;
                if (scale != 0.0f) {
                    float x = (float)row_exact[h];
                    float v = x / scale;
                    code = (uint8_t)oracle_encode(ORC_E4M3, (double)v);
                }
                q_out[t * H + h] = code;
            }
        }
    }
    free(row_exact);
    free(row_norm);
    return rc;
}

int oracle_ar_rms_quant(int W, int64_t T, int64_t H, int f,
                        const uint16_t *const *partials, const uint16_t *residual,
                        const uint16_t *weight, float eps, int gemma, int64_t group,
                        uint16_t *norm_out, uint8_t *q_out, float *scales,
                        uint16_t *residual_out, double *exact)
{
    return oracle_ar_rms_quant_ex(W, T, H, f, partials, residual, weight, eps, gemma, 0, group,
                                  norm_out, q_out, scales, residual_out, exact);
}

/* ------------------------------------------------------------------------- */
/* QK-norm across W shards                                                    */
/* ------------------------------------------------------------------------- */

/* Shard r holds rows of `stride` elements laid out [q | k | v] (q_size, kv_size,
 * kv_size).  For every token t:
 *   ssq = sum_r sum_{j<q_size} x_r[t,j]^2,          rq = 1/sqrt(ssq/(W*q_size) + eps)
 *   ssk = sum_r sum_{j<kv_size} x_r[t,q_size+j]^2,  rk = 1/sqrt(ssk/(W*kv_size) + eps)
 *   q_out[r,t,j] = round(x_r[t,j] * rq * q_w[r*q_size + j])
 *   k_out[r,t,j] = round(x_r[t,q_size+j] * rk * k_w[r*kv_size + j])
 * which is the RMSNorm of the concatenation of the W shards' q (k) heads over the
 * full head dimension.  v is neither read nor written.  q_exact / k_exact may be
 * NULL. */
int oracle_qknorm(int W, int64_t T, int64_t q_size, int64_t kv_size, int64_t stride, int f,
                  const uint16_t *const *qkv, const uint16_t *q_w, const uint16_t *k_w,
                  float eps, uint16_t *q_out, uint16_t *k_out,
                  double *q_exact, double *k_exact)
{
    if (W < 1 || T < 0 || q_size <= 0 || kv_size <= 0 || stride < q_size + kv_size ||
        (f != ORC_BF16 && f != ORC_FP16))
        return -1;
    for (int64_t t = 0; t < T; ++t) {
        double ssq = 0.0, ssk = 0.0;
        for (int r = 0; r < W; ++r) {
            const uint16_t *x = qkv[r] + t * stride;
            for (int64_t j = 0; j < q_size; ++j) {
                double v = oracle_decode(f, x[j]);
                ssq += v * v;
            }
            for (int64_t j = 0; j < kv_size; ++j) {
                double v = oracle_decode(f, x[q_size + j]);
                ssk += v * v;
            }
        }
        double rq = 1.0 / sqrt(ssq / (double)(W * q_size) + (double)eps);
        double rk = 1.0 / sqrt(ssk / (double)(W * kv_size) + (double)eps);
        for (int r = 0; r < W; ++r) {
            const uint16_t *x = qkv[r] + t * stride;
            for (int64_t j = 0; j < q_size; ++j) {
                double y = oracle_decode(f, x[j]) * rq * oracle_decode(f, q_w[r * q_size + j]);
                int64_t o = ((int64_t)r * T + t) * q_size + j;
                if (q_exact) q_exact[o] = y;
                q_out[o] = (uint16_t)oracle_encode(f, y);
            }
            for (int64_t j = 0; j < kv_size; ++j) {
                double y = oracle_decode(f, x[q_size + j]) * rk *
                           oracle_decode(f, k_w[r * kv_size + j]);
                int64_t o = ((int64_t)r * T + t) * kv_size + j;
                if (k_exact) k_exact[o] = y;
                k_out[o] = (uint16_t)oracle_encode(f, y);
            }
        }
    }
    return 0;
}
