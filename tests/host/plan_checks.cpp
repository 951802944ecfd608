// Exercises the host-only part of libarrms (plans, the one-stage predicate and
// the argument checks) over valid, boundary and extreme arguments, for a build
// with AddressSanitizer and UndefinedBehaviorSanitizer.  Checks invariants the
// header states; the exact status of each case is pinned by the Python tests.
// Addresses are never dereferenced: the checks only look at their values.
#include <cinttypes>
#include <cstdio>
#include <cstring>

#include "../../tp_all_reduce_amd/csrc/arrms_host.h"

namespace {
int failures = 0;

void expect(bool ok, const char *what, long long a = 0, long long b = 0, long long c = 0) {
    if (!ok) {
        ++failures;
        std::fprintf(stderr, "FAIL %s (%lld, %lld, %lld): %s\n", what, a, b, c,
                     ar_rms_last_error());
    }
}

bool known_status(int rc) {
    return rc == ARRMS_OK || rc == ARRMS_EINVAL || rc == ARRMS_ENOTSUP || rc == ARRMS_EHIP ||
           rc == ARRMS_ENOMEM;
}

const void *addr(uintptr_t a) { return reinterpret_cast<const void *>(a); }
}  // namespace

int main() {
    const int Ws[] = {-1, 0, 1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 64, 1 << 30};
    const int64_t Ts[] = {-1, 0, 1, 8, 21, 22, 31, 32, 80, 81, 1000, int64_t(1) << 40, INT64_MAX};
    const int64_t Hs[] = {-8, 0, 7, 8, 1000, 1020, 4096, 6144, 7168, 8192, 8193, 8200,
                          16384, 16392, int64_t(1) << 40, INT64_MAX};
    const int dtypes[] = {-1, ARRMS_BF16, ARRMS_FP16, 2};
    const uint32_t flagss[] = {0u, 1u, 2u, 3u, 4u, 5u, 6u, 8u, 0xffffffffu};
    long plans = 0;
    for (int W : Ws)
        for (int64_t T : Ts)
            for (int64_t H : Hs)
                for (int dt : dtypes) {
                    const int one = ar_rms_one_stage(W, T, H, dt, 1);
                    expect(one == 0 || one == 1, "predicate is 0 or 1", W, T, H);
                    if (one) expect(W >= 1 && W <= 8 && T <= 80 && H % 8 == 0 && H <= 8192,
                                    "predicate window", W, T, H);
                    expect(ar_rms_one_stage(W, T, H, dt, 0) <= one, "topology only narrows", W, T, H);
                    for (uint32_t f : flagss) {
                        ar_rms_plan_t p = reinterpret_cast<ar_rms_plan_t>(1);
                        const int rc = ar_rms_plan(W, T, H, dt, f, &p);
                        expect(known_status(rc), "status", W, T, H);
                        expect(std::strlen(ar_rms_last_error()) < 512, "message length", W, T, H);
                        if (rc != ARRMS_OK) {
                            expect(p == nullptr, "no plan on error", W, T, H);
                            expect(ar_rms_last_error()[0] != '\0', "message on error", W, T, H);
                            continue;
                        }
                        ++plans;
                        expect(p != nullptr, "plan on success", W, T, H);
                        expect(W >= 1 && W <= 16 && T >= 0 && H % 8 == 0 && H <= 16384 &&
                                   (dt == ARRMS_BF16 || dt == ARRMS_FP16) && (f & ~7u) == 0,
                               "accepted arguments", W, T, H);
                        expect(W <= 8 || H <= 8192, "more than eight partials: short rows", W, T, H);
                        const int k = ar_rms_plan_kernel(p);
                        expect(k == ARRMS_KERNEL_ROW || k == ARRMS_KERNEL_SPLIT, "kernel", W, T, H);
                        if (f & ARRMS_FORCE_ROW) expect(k == ARRMS_KERNEL_ROW, "forced row", W, T, H);
                        if (f & ARRMS_FORCE_SPLIT) expect(k == ARRMS_KERNEL_SPLIT, "forced split", W, T, H);
                        if (!(f & 3u)) expect((k == ARRMS_KERNEL_ROW) == (one == 1), "default kernel", W, T, H);
                        const int packs = int(H / 8);
                        expect(p->block % 64 == 0 && p->block >= 64 && p->block <= 1024, "block", W, T, H);
                        expect(p->ppl == 1 || p->ppl == 4, "packs per lane", W, T, H);
                        expect(int64_t(p->block) * p->ppl >= packs, "lanes cover the row", W, T, H);
                        expect(p->block - 64 < (packs + p->ppl - 1) / p->ppl, "no idle wavefront", W, T, H);
                        ar_rms_plan_destroy(p);
                    }
                }
    ar_rms_plan_destroy(nullptr);
    expect(ar_rms_plan(2, 8, 1024, ARRMS_BF16, 0, nullptr) == ARRMS_EINVAL, "out NULL");
    expect(ar_rms_plan_kernel(nullptr) == ARRMS_EINVAL, "kernel of NULL");

    // argument checks: aligned fake addresses pass, each misalignment or NULL fails
    ar_rms_plan_t p = nullptr;
    expect(ar_rms_plan(3, 8, 1024, ARRMS_BF16, 0, &p) == ARRMS_OK, "plan for checks");
    const uintptr_t A = 0x10000;
    const void *parts[3] = {addr(A), addr(A + 0x1000), addr(A + 0x2000)};
    const void *bad_parts[3] = {addr(A), addr(A + 8), addr(A + 0x2000)};
    const void *null_parts[3] = {addr(A), nullptr, addr(A + 0x2000)};
    using arrms::check_rms_args;
    expect(check_rms_args(p, parts, addr(A), addr(A), 1e-6f, addr(A), true, addr(A)) == 0, "valid rms");
    expect(check_rms_args(p, parts, nullptr, addr(A), 1e-6f, addr(A), true, nullptr) == 0, "no residual");
    expect(check_rms_args(p, bad_parts, addr(A), addr(A), 1e-6f, addr(A), true, addr(A)) == ARRMS_EINVAL, "misaligned partial");
    expect(check_rms_args(p, null_parts, addr(A), addr(A), 1e-6f, addr(A), true, addr(A)) == ARRMS_EINVAL, "NULL partial");
    expect(check_rms_args(p, nullptr, addr(A), addr(A), 1e-6f, addr(A), true, addr(A)) == ARRMS_EINVAL, "NULL array");
    expect(check_rms_args(p, parts, addr(A + 2), addr(A), 1e-6f, addr(A), true, addr(A)) == ARRMS_EINVAL, "misaligned residual");
    expect(check_rms_args(p, parts, addr(A), nullptr, 1e-6f, addr(A), true, addr(A)) == ARRMS_EINVAL, "NULL weight");
    expect(check_rms_args(p, parts, addr(A), addr(A), 1e-6f, nullptr, true, addr(A)) == ARRMS_EINVAL, "NULL norm_out");
    expect(check_rms_args(p, parts, addr(A), addr(A), 1e-6f, nullptr, false, addr(A)) == 0, "norm_out optional");
    expect(check_rms_args(p, parts, addr(A), addr(A), 1e-6f, addr(A), true, addr(A + 4)) == ARRMS_EINVAL, "misaligned residual_out");
    const float bad_eps[] = {-1.0f, __builtin_nanf(""), __builtin_inff(), -__builtin_inff()};
    for (float e : bad_eps)
        expect(check_rms_args(p, parts, addr(A), addr(A), e, addr(A), true, addr(A)) == ARRMS_EINVAL, "bad eps");
    expect(check_rms_args(nullptr, parts, addr(A), addr(A), 1e-6f, addr(A), true, addr(A)) == ARRMS_EINVAL, "NULL plan");
    using arrms::check_quant_args;
    const int groups[] = {-8, 0, 4, 8, 16, 96, 128, 256, 512, 1024, 1 << 30};
    for (int g : groups) {
        const int rc = check_quant_args(p, g, addr(A), addr(A));
        const bool ok = g >= 8 && g <= 512 && (g & (g - 1)) == 0 && 1024 % g == 0;
        expect(rc == (ok ? 0 : ARRMS_ENOTSUP), "group size", g);
    }
    expect(check_quant_args(p, 128, addr(A + 4), addr(A)) == ARRMS_EINVAL, "misaligned codes");
    expect(check_quant_args(p, 128, addr(A), addr(A + 2)) == ARRMS_EINVAL, "misaligned scales");
    ar_rms_plan_destroy(p);

    using arrms::check_qk_args;
    ar_rms_plan_t q = nullptr;
    expect(ar_rms_plan(4, 64, 2048, ARRMS_BF16, 0, &q) == ARRMS_OK, "QK plan");
    const void *shards[4] = {addr(A), addr(A + 0x1000), addr(A + 0x2000), addr(A + 0x3000)};
    expect(check_qk_args(q, shards, 1536, 256, addr(A), addr(A), 1e-6f, addr(A), addr(A)) == 0, "valid QK");
    const int sizes[][2] = {{0, 256}, {-256, 256}, {1536, 0}, {1792, 128}, {1024, 256},
                            {1 << 30, 1 << 30}, {2147483392, 256}, {256, 2147483392}};
    for (const auto &qs : sizes) {
        const int rc = check_qk_args(q, shards, qs[0], qs[1], addr(A), addr(A), 1e-6f, addr(A), addr(A));
        expect(rc == ARRMS_EINVAL || rc == ARRMS_ENOTSUP, "bad QK sizes", qs[0], qs[1]);
    }
    expect(check_qk_args(q, shards, 1536, 256, addr(A + 8), addr(A), 1e-6f, addr(A), addr(A)) == ARRMS_EINVAL, "misaligned q_weight");
    expect(check_qk_args(q, shards, 1536, 256, addr(A), addr(A), 1e-6f, addr(A), nullptr) == ARRMS_EINVAL, "NULL k_out");
    ar_rms_plan_destroy(q);
    ar_rms_plan_t many = nullptr;
    expect(ar_rms_plan(9, 64, 768, ARRMS_BF16, 0, &many) == ARRMS_OK, "W=9 plan");
    const void *nine[9] = {};
    expect(check_qk_args(many, nine, 256, 256, addr(A), addr(A), 1e-6f, addr(A), addr(A)) == ARRMS_ENOTSUP, "QK W > 8");
    ar_rms_plan_destroy(many);

    // QK lane layouts: shards on whole wavefronts when that fits one workgroup
    long aligned = 0, packed = 0;
    for (int W = 1; W <= 8; ++W)
        for (int q = 256; q <= 32768; q += 256)
            for (int kv = 256; kv <= 32768; kv += 256) {
                if (int64_t(W) * (q + kv) > 32768) continue;
                const arrms::Shape a = arrms::qk_aligned_shape(W, q, kv);
                const arrms::Shape b = arrms::qk_shape(W, q, kv);
                const int per_shard = (q + kv) / 8;
                expect(b.block % 64 == 0 && b.block <= 1024 && int64_t(b.block) * b.ppl >= W * per_shard,
                       "packed shape", W, q, kv);
                if (a.block == 0) { ++packed; continue; }
                ++aligned;
                const int lanes = a.block / W;
                expect(a.block % W == 0 && lanes % 64 == 0 && a.block <= 1024, "aligned block", W, q, kv);
                expect(a.ppl == 1 || a.ppl == 2 || a.ppl == 4, "aligned ppl", W, q, kv);
                expect(int64_t(lanes) * a.ppl >= per_shard && lanes - 64 < (per_shard + a.ppl - 1) / a.ppl,
                       "aligned lanes cover a shard", W, q, kv);
                // the fewest packs per lane that fit, except that four or more
                // shards filling 1024 lanes at one pack per lane take two
                int want = 0;
                for (int ppl = 1; ppl <= 4 && want == 0; ppl *= 2) {
                    const int l = ((per_shard + ppl - 1) / ppl + 63) / 64 * 64;
                    if (W * l > 1024 || (ppl == 1 && W >= 4 && W * l == 1024)) continue;
                    want = ppl;
                }
                expect(a.ppl == want, "aligned ppl choice", W, q, kv);
            }
    expect(aligned > 0 && packed > 0, "both QK layouts occur", aligned, packed);

    std::printf("%s: %ld plans built, %d failures\n", failures ? "FAILED" : "OK", plans, failures);
    return failures ? 1 : 0;
}
