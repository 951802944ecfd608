// A C++ caller of libarrms with no Python in the path: device memory and a
// stream from the HIP runtime, calls through include/arrms.h only, outputs
// checked against the C oracle (test infrastructure, linked here as a test
// program may be) with the same acceptance rules as the Python parity tests:
// residual_out bit-exact, norm and q/k outputs within 4e-3 relative (bf16) of
// the oracle's fp64 value, FP8 codes within one step, scales within 1e-6.
//
// Exit status: 0 all cases match, 1 a mismatch or a library error, 77 no GPU.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "arrms.h"

extern "C" {
double oracle_decode(int f, uint32_t bits);
int oracle_ar_rms_ex(int W, int64_t T, int64_t H, int f, const uint16_t *const *partials,
                     const uint16_t *residual, const uint16_t *weight, float eps, int gemma,
                     int round_reduced, uint16_t *norm_out, uint16_t *residual_out,
                     double *exact);
int oracle_ar_rms_quant_ex(int W, int64_t T, int64_t H, int f, const uint16_t *const *partials,
                           const uint16_t *residual, const uint16_t *weight, float eps,
                           int gemma, int round_reduced, int64_t group, uint16_t *norm_out,
                           uint8_t *q_out, float *scales, uint16_t *residual_out,
                           double *exact);
int oracle_qknorm(int W, int64_t T, int64_t q_size, int64_t kv_size, int64_t stride, int f,
                  const uint16_t *const *qkv, const uint16_t *q_w, const uint16_t *k_w,
                  float eps, uint16_t *q_out, uint16_t *k_out, double *q_exact,
                  double *k_exact);
}

namespace {

constexpr int kBf16 = 0;          // the oracle's code for bfloat16
constexpr double kTol = 4e-3;     // bf16 acceptance for norm / q / k outputs
int failures = 0;

void fail(const char *what) {
    ++failures;
    std::fprintf(stderr, "FAIL %s (%s)\n", what, ar_rms_last_error());
}

void check_hip(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        std::fprintf(stderr, "HIP error in %s: %s\n", what, hipGetErrorString(e));
        std::exit(1);
    }
}

// Deterministic bf16 inputs: a 64-bit LCG, values mean + std * (sum of four
// uniforms - 2) * sqrt(3), rounded to bf16 by nearest-even on the float bits.
struct Inputs {
    uint64_t state;
    explicit Inputs(uint64_t seed) : state(seed * 6364136223846793005ull + 1442695040888963407ull) {}
    double uniform() {
        state = state * 6364136223846793005ull + 1442695040888963407ull;
        return double(state >> 11) * (1.0 / 9007199254740992.0);
    }
    uint16_t bf16(double mean, double std) {
        const double z = (uniform() + uniform() + uniform() + uniform() - 2.0) * std::sqrt(3.0);
        const float v = float(mean + std * z);
        uint32_t u;
        std::memcpy(&u, &v, 4);
        u += 0x7fffu + ((u >> 16) & 1u);
        return uint16_t(u >> 16);
    }
    std::vector<uint16_t> fill(size_t n, double mean, double std) {
        std::vector<uint16_t> v(n);
        for (auto &x : v) x = bf16(mean, std);
        return v;
    }
};

template <typename T>
T *to_device(const std::vector<T> &h) {
    T *d = nullptr;
    check_hip(hipMalloc(&d, h.size() * sizeof(T) + 16), "hipMalloc");
    check_hip(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice), "copy in");
    return d;
}

template <typename T>
std::vector<T> to_host(const T *d, size_t n) {
    std::vector<T> h(n);
    check_hip(hipMemcpy(h.data(), d, n * sizeof(T), hipMemcpyDeviceToHost), "copy out");
    return h;
}

double max_relerr(const std::vector<uint16_t> &got, const std::vector<double> &exact) {
    const double min_normal = std::ldexp(1.0, -126);
    double worst = 0.0;
    for (size_t i = 0; i < got.size(); ++i) {
        const double g = oracle_decode(kBf16, got[i]);
        const double e = exact[i];
        const double err = std::fabs(g - e) / std::fmax(std::fabs(e), min_normal);
        if (!(err <= worst)) worst = err;   // NaN counts as the worst
    }
    return worst;
}

int code_rank(uint8_t c) { return (c & 0x80) ? -int(c & 0x7f) : int(c & 0x7f); }

// reduce + residual add + RMSNorm (optionally the FP8 epilogue), W x [T, H]
void rms_case(const char *name, int W, int64_t T, int64_t H, uint32_t flags, int gemma,
              int group, hipStream_t s, uint64_t seed) {
    Inputs gen(seed);
    const size_t n = size_t(T) * size_t(H);
    std::vector<std::vector<uint16_t>> P;
    for (int r = 0; r < W; ++r) P.push_back(gen.fill(n, 0.0, 1.0));
    const std::vector<uint16_t> R = gen.fill(n, 0.0, 1.0);
    const std::vector<uint16_t> w = gen.fill(size_t(H), gemma ? 0.0 : 1.0, 0.1);

    std::vector<uint16_t *> dP;
    std::vector<const void *> ptrs;
    for (auto &p : P) {
        dP.push_back(to_device(p));
        ptrs.push_back(dP.back());
    }
    uint16_t *dR = to_device(R), *dw = to_device(w);
    uint16_t *dN = to_device(std::vector<uint16_t>(n, 0)), *dRo = to_device(std::vector<uint16_t>(n, 0));
    const int64_t groups = group ? H / group : 0;
    uint8_t *dQ = group ? to_device(std::vector<uint8_t>(n, 0)) : nullptr;
    float *dS = group ? to_device(std::vector<float>(size_t(T) * groups, 0.0f)) : nullptr;

    ar_rms_plan_t plan = nullptr;
    if (ar_rms_plan(W, T, H, ARRMS_BF16, flags, &plan) != ARRMS_OK) return fail(name);
    const float eps = 1e-6f;
    const int rc = group ? ar_rms_quant_run(plan, ptrs.data(), dR, dw, eps, gemma, group, dN, dQ,
                                            dS, dRo, s)
                         : ar_rms_run(plan, ptrs.data(), dR, dw, eps, gemma, dN, dRo, s);
    ar_rms_plan_destroy(plan);
    if (rc != ARRMS_OK) return fail(name);
    check_hip(hipStreamSynchronize(s), "sync");

    std::vector<const uint16_t *> hp;
    for (auto &p : P) hp.push_back(p.data());
    std::vector<uint16_t> on(n), ores(n);
    std::vector<double> exact(n);
    const int round_reduced = (flags & ARRMS_ROUND_REDUCED) ? 1 : 0;
    std::vector<uint8_t> oq(group ? n : 0);
    std::vector<float> os(group ? size_t(T) * groups : 0);
    if (group)
        oracle_ar_rms_quant_ex(W, T, H, kBf16, hp.data(), R.data(), w.data(), eps, gemma,
                               round_reduced, group, on.data(), oq.data(), os.data(), ores.data(),
                               exact.data());
    else
        oracle_ar_rms_ex(W, T, H, kBf16, hp.data(), R.data(), w.data(), eps, gemma, round_reduced,
                         on.data(), ores.data(), exact.data());

    if (to_host(dRo, n) != ores) fail(name);                      // residual_out bit-exact
    const double err = max_relerr(to_host(dN, n), exact);
    if (!(err <= kTol)) fail(name);
    if (group) {
        const std::vector<uint8_t> q = to_host(dQ, n);
        for (size_t i = 0; i < n; ++i)
            if (std::abs(code_rank(q[i]) - code_rank(oq[i])) > 1) { fail(name); break; }
        const std::vector<float> sc = to_host(dS, os.size());
        for (size_t i = 0; i < sc.size(); ++i) {
            const double den = os[i] == 0.0f ? 1.0 : std::fabs(double(os[i]));
            if (std::fabs(double(sc[i]) - double(os[i])) / den > 1e-6) { fail(name); break; }
        }
    }
    std::printf("%-44s norm relerr %.3e\n", name, err);
    for (auto *d : dP) (void)hipFree(d);
    (void)hipFree(dR); (void)hipFree(dw); (void)hipFree(dN); (void)hipFree(dRo);
    if (dQ) (void)hipFree(dQ);
    if (dS) (void)hipFree(dS);
}

// QK-norm across W shards [T, q + 2 kv]
void qk_case(const char *name, int W, int64_t T, int q, int kv, hipStream_t s, uint64_t seed) {
    Inputs gen(seed);
    const int64_t H = q + 2 * kv;
    std::vector<std::vector<uint16_t>> X;
    for (int r = 0; r < W; ++r) X.push_back(gen.fill(size_t(T) * H, 0.0, 1.0));
    const std::vector<uint16_t> qw = gen.fill(size_t(W) * q, 1.0, 0.1);
    const std::vector<uint16_t> kw = gen.fill(size_t(W) * kv, 1.0, 0.1);
    std::vector<uint16_t *> dX;
    std::vector<const void *> ptrs;
    for (auto &x : X) {
        dX.push_back(to_device(x));
        ptrs.push_back(dX.back());
    }
    uint16_t *dqw = to_device(qw), *dkw = to_device(kw);
    const size_t nq = size_t(W) * T * q, nk = size_t(W) * T * kv;
    uint16_t *dqo = to_device(std::vector<uint16_t>(nq, 0)), *dko = to_device(std::vector<uint16_t>(nk, 0));
    ar_rms_plan_t plan = nullptr;
    if (ar_rms_plan(W, T, H, ARRMS_BF16, 0, &plan) != ARRMS_OK) return fail(name);
    const float eps = 1e-6f;
    const int rc = ar_qknorm_run(plan, ptrs.data(), q, kv, dqw, dkw, eps, dqo, dko, s);
    ar_rms_plan_destroy(plan);
    if (rc != ARRMS_OK) return fail(name);
    check_hip(hipStreamSynchronize(s), "sync");
    std::vector<const uint16_t *> hx;
    for (auto &x : X) hx.push_back(x.data());
    std::vector<uint16_t> oq(nq), ok(nk);
    std::vector<double> eq(nq), ek(nk);
    oracle_qknorm(W, T, q, kv, H, kBf16, hx.data(), qw.data(), kw.data(), eps, oq.data(),
                  ok.data(), eq.data(), ek.data());
    const double e1 = max_relerr(to_host(dqo, nq), eq), e2 = max_relerr(to_host(dko, nk), ek);
    if (!(e1 <= kTol) || !(e2 <= kTol)) fail(name);
    std::printf("%-44s q relerr %.3e, k relerr %.3e\n", name, e1, e2);
    for (auto *d : dX) (void)hipFree(d);
    (void)hipFree(dqw); (void)hipFree(dkw); (void)hipFree(dqo); (void)hipFree(dko);
}

}  // namespace

int main() {
    int devices = 0;
    if (hipGetDeviceCount(&devices) != hipSuccess || devices == 0) {
        std::printf("no GPU\n");
        return 77;
    }
    check_hip(hipSetDevice(0), "hipSetDevice");
    hipStream_t s;
    check_hip(hipStreamCreate(&s), "hipStreamCreate");
    rms_case("decode W=4 [8, 4096] Gemma, row kernel", 4, 8, 4096, ARRMS_FORCE_ROW, 1, 0, s, 1);
    rms_case("prefill W=8 [600, 8192], split kernel loops", 8, 600, 8192, 0, 0, 0, s, 2);
    rms_case("W=4 [8, 4096], unfused numerics", 4, 8, 4096, ARRMS_ROUND_REDUCED, 0, 0, s, 3);
    rms_case("FP8 groups of 128, W=4 [16, 7168]", 4, 16, 7168, 0, 0, 128, s, 4);
    rms_case("W=12 [40, 2048] (more than eight partials)", 12, 40, 2048, 0, 0, 0, s, 5);
    qk_case("QK-norm W=4 [4, 1536 + 256 + 256]", 4, 4, 1536, 256, s, 6);
    check_hip(hipStreamDestroy(s), "hipStreamDestroy");
    std::printf("%s: %d failures\n", failures ? "FAILED" : "OK", failures);
    return failures ? 1 : 0;
}
