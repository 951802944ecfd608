// HIP kernels (gfx950, wave64) of libarrms, with their launchers and the
// templates that pick a variant.  Every kernel unit includes this header and
// instantiates one slice of the variants; all definitions here have internal
// linkage, so each unit holds only the kernels it picks.
//
// The fused tensor-parallel layer epilogue of the vLLM PR #54787 page
// ("Motivation"; "Key source excerpts": fused_allreduce_gemma_rms_norm and
// _rocm_aiter_fused_allreduce_rmsnorm_impl), on one GPU: W partial-sum
// buffers [T, H] stand in for the W ranks' buffers and are reduced in the
// kernel.  Per token row:
//   phase 1  16-byte loads of all W partials and the residual, fp32 sum in
//            rank order with the residual last, residual_out store, per-lane
//            sum of squares;
//   reduce   wave64 sum with DPP row ops plus readlane, one LDS exchange and
//            one barrier across the workgroup's wavefronts;
//   phase 2  rstd, (1 + w) or w, 16-bit norm_out store, and optionally the
//            per-group FP8 epilogue (group amax by DPP within the lanes that
//            hold the group, scale = amax / 448, E4M3FN codes by the hardware
//            conversion).
// The row stays in registers between the phases, so HBM sees each input once
// and each output once: (W + 3) * T * H * 2 bytes (W partials and the residual
// read, residual_out and norm_out written) plus the weight.
//
// Kernel bodies (the plan picks the launch; see Mode in launch.h):
//   row        one workgroup per token row, one 16-byte pack per lane (up to
//              1024 lanes = 8192 elements), straight-line code; lowest
//              latency for the decode window, where the launch and one DRAM
//              round trip are the whole cost;
//   split      a persistent grid sized to what the CUs hold at once; each
//              workgroup loops over rows and issues the next row's loads
//              before it reduces and normalises the current one, so HBM
//              stays busy through the barrier and the epilogue;
//   split-wide persistent without the row-ahead loads, for rows that leave
//              no registers for a second row (longer than 8192 elements, or
//              more than eight partials), and, with one pack per lane (the
//              lean mode), for split plans of only a few rows per workgroup:
//              its registers leave room for two workgroups per CU.
// The looping bodies stream partials and residual with non-temporal loads
// (read once) and write their outputs at device scope, through the XCDs' L2
// caches; the row body stores residual_out, next read a layer later, with the
// non-temporal hint (reduce_norm states the store policy of each body).  The
// weight row is loaded once per workgroup and kept in registers (split-wide
// with one pack per lane keeps it in LDS; with four, reloads it per row from
// L2).
//
// There is no inter-workgroup communication, no atomics and no scratch
// memory: every output is a fixed function of the inputs and bit-identical
// from run to run.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace arrms {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct Bf16 {};
struct Fp16 {};

// Two 16-bit elements per dword, element 0 in the low half.
template <typename IO>
struct Codec;

template <>
struct Codec<Bf16> {
    static __device__ __forceinline__ f32x2 unpack(uint32_t u) {
        return f32x2{__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
    }
    // v_cvt_pk_bf16_f32: round to nearest even
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
    }
};

template <>
struct Codec<Fp16> {
    static __device__ __forceinline__ f32x2 unpack(uint32_t u) {
        return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
    }
    // v_cvt_pk_f16_f32: round to nearest even
    static __device__ __forceinline__ uint32_t pack(float a, float b) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
    }
};

template <typename IO>
__device__ __forceinline__ void unpack8(u32x4 v, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f32x2 p = Codec<IO>::unpack(v[i]);
        x[2 * i] = p.x;
        x[2 * i + 1] = p.y;
    }
}

template <typename IO>
__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = Codec<IO>::pack(x[2 * i], x[2 * i + 1]);
    return v;
}

__device__ __forceinline__ u32x4 load16(const uint8_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

// Streaming load: the data is read exactly once.
__device__ __forceinline__ u32x4 load16_stream(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void store16(uint8_t *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Streaming store (non-temporal hint).
__device__ __forceinline__ void store16_stream(uint8_t *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Cache policy of an output store, as the bits of the cache-policy operand of
// a gfx950 buffer store: bit 1 the non-temporal hint, bit 4 device scope (the
// store is written through the XCD's L2 rather than left there dirty, to be
// written back when it is evicted or when the kernel ends).
enum StorePolicy {
    kStorePlain = 0,
    kStoreStream = 2,
    kStoreDevice = 16,
    kStoreDeviceStream = 16 | 2,
};

// Word 3 of a raw buffer resource: 32-bit data format, the setting untyped
// buffer accesses expect on gfx9-family GPUs.
constexpr int kRawBufferWord3 = 0x00020000;

// 16-byte store of one lane's pack at `off` bytes past a wave-uniform `base`
// (a row of `bytes` bytes) with the given cache policy.  Plain and
// non-temporal stores are global stores; the device-scope ones are buffer
// stores, whose resource (in scalar registers) holds the row's base and
// length, so a store past the row would be dropped by the hardware.
template <int POLICY>
__device__ __forceinline__ void store16_policy(uint8_t *base, uint32_t off, uint32_t bytes,
                                               u32x4 v) {
    if constexpr (POLICY == kStorePlain) {
        store16(base + off, v);
    } else if constexpr (POLICY == kStoreStream) {
        store16_stream(base + off, v);
    } else {
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(base, 0, int(bytes), kRawBufferWord3);
        __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, POLICY);
    }
}

// ---------------------------------------------------------------- wave64 ops
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141; // row_half_mirror: lane i <-> 7-i within 8 lanes
constexpr int kRowMirror = 0x140;  // row_mirror: lane i <-> 15-i within 16 lanes

// Sum over each 16-lane row; every lane of the row ends with the same bits
// (each step adds a value to its mirror image, which is commutative).
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    v += dpp<kHalfMirror>(v);
    v += dpp<kRowMirror>(v);
    return v;
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Wave-uniform sum over all 64 lanes (all lanes must be active).
__device__ __forceinline__ float wave_sum(float v) {
    v = row16_sum(v);
    return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}

// Sum of the first n (<= 16) per-wavefront partials in LDS, the same bits in
// every lane.  Beyond eight: lane i reads partial i mod 16 (0 from n on) and
// the 16-lane DPP sum adds them in a fixed tree order, one LDS read and one
// wait where a loop would read and wait per group of partials.
__device__ __forceinline__ float sum_wave_partials(const float *ws, int n, int lane) {
    if (n <= 8) {
        // few partials: broadcast reads in index order cost less than the DPP
        float t = 0.0f;
        for (int i = 0; i < n; ++i) t += ws[i];
        return t;
    }
    const int i = lane & 15;
    return row16_sum(i < n ? ws[i] : 0.0f);
}

// The q and k statistics of QK-norm: the sums of the first n (<= 16) entries of
// `a` and of `b`, the same bits in every lane.  Lane i reads entry i mod 16 of
// both (0 from n on), so both LDS reads are in flight together and the two
// 16-lane DPP sums interleave: for two statistics this measured faster than two
// index-order loops, each with its own LDS round trip.  Both arrays hold 16
// entries.
__device__ __forceinline__ f32x2 sum_wave_partials2(const float *a, const float *b, int n,
                                                   int lane) {
    const int i = lane & 15;
    const float x = a[i];
    const float y = b[i];
    return f32x2{row16_sum(i < n ? x : 0.0f), row16_sum(i < n ? y : 0.0f)};
}

// The group maxima below take per-lane maxima of magnitudes: non-negative
// floats that are never NaN (a lane's maximum starts at 0 and fmaxf skips NaN).
// On those, the order of the bit patterns as unsigned integers is the order of
// the values, so each step is one unsigned max with a DPP operand; a float max
// would first quiet its operands (three instructions and a move per step).
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t v) {
    const uint32_t o = uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
    return v > o ? v : o;
}

__device__ __forceinline__ uint32_t umax_xor(uint32_t v, int lane_mask) {
    const uint32_t o = uint32_t(__shfl_xor(int(v), lane_mask));
    return v > o ? v : o;
}

// Max over aligned groups of 16 consecutive lanes (128-element groups of 16-bit
// data), in straight-line code.
__device__ __forceinline__ float group_max16(float v) {
    uint32_t u = __float_as_uint(v);
    u = umax_dpp<kQuadSwap1>(u);
    u = umax_dpp<kQuadSwap2>(u);
    u = umax_dpp<kHalfMirror>(u);
    return __uint_as_float(umax_dpp<kRowMirror>(u));
}

// Max over aligned groups of `lanes` consecutive lanes (1..64, a power of two);
// every lane of a group ends with the group's max.  The common 16-lane group
// takes one uniform branch instead of a test per step.
__device__ __forceinline__ float group_max(float v, int lanes) {
    if (lanes == 16) return group_max16(v);
    uint32_t u = __float_as_uint(v);
    if (lanes >= 2) u = umax_dpp<kQuadSwap1>(u);
    if (lanes >= 4) u = umax_dpp<kQuadSwap2>(u);
    if (lanes >= 8) u = umax_dpp<kHalfMirror>(u);
    if (lanes >= 16) u = umax_dpp<kRowMirror>(u);
    if (lanes >= 32) u = umax_xor(u, 16);
    if (lanes >= 64) u = umax_xor(u, 32);
    return __uint_as_float(u);
}

// amax / 448 correctly rounded, in three instructions where the quotient is a
// normal number: the product with c = RN(1/448) and one FMA correction equal the
// IEEE quotient for every such input (checked over every float on the CPU, and
// by the CPU tests over the binades at the guard); below 2^-116, where some
// subnormal quotients differ, and for inf, the division.
__device__ __forceinline__ float div448(float amax) {
    if (amax >= 0x1p-116f && amax <= 3.40282347e38f) {
        const float c = 1.0f / 448.0f;
        const float q = amax * c;
        return __builtin_fmaf(__builtin_fmaf(-q, 448.0f, amax), c, q);
    }
    return amax / 448.0f;
}

// Four fp32 values -> four OCP FP8 E4M3FN codes (byte i = value i), rounded to
// nearest even by v_cvt_pk_fp8_f32.  The instruction turns magnitudes that
// round beyond 448 into NaN (and NaN into 0xFF); the callers only pass values
// of magnitude <= 448 * (1 + 2^-22), which round to at most 448.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// ------------------------------------------------------- reduce + RMSNorm
// Issues the loads of one row: W partial packs and (RES) the residual pack for
// each of the lane's PPL packs (pack pk = lane + k * workgroup size), with the
// non-temporal hint in the looping (large-T) bodies; the row body's inputs are
// small and may still be cached from the op that wrote them.  A lane
// past the row's end loads pack 0 of the row instead (its sum is zeroed and
// nothing of it is stored): with no branch around a load, the compiler places
// no wait at a join.
template <int W, int PPL, bool RES, bool STREAM>
__device__ __forceinline__ void load_row(const RmsParams &p, int64_t row, int tid, int nthr,
                                         u32x4 (&v)[PPL][W + RES]) {
    const size_t base = size_t(row) * size_t(p.H) * 2;
#pragma unroll
    for (int k = 0; k < PPL; ++k) {
        const int pk = tid + k * nthr;
        const size_t off = base + size_t(pk < p.packs ? pk : 0) * 16;
#pragma unroll
        for (int r = 0; r < W; ++r)
            v[k][r] = STREAM ? load16_stream(p.partials[r] + off) : load16(p.partials[r] + off);
        if constexpr (RES)
            v[k][W] = STREAM ? load16_stream(p.residual + off) : load16(p.residual + off);
    }
    // Keep every load ahead of what follows: the scheduler would otherwise put
    // one behind the wait for the scalar load of the output pointers.
    __builtin_amdgcn_sched_barrier(0);
}

// One pack per lane: up to 1024 lanes.  Several packs per lane (rows longer
// than 1024 packs): up to 512 lanes, which leaves 256 registers per lane.
constexpr int rms_block_bound(int ppl) { return ppl == 1 ? kMaxBlock : kMaxBlock / 2; }

// RES: a residual term is present (compile-time, so that every load of a row
// is issued before the first wait).  ROUND: the W-way sum is rounded to the
// I/O format before the residual add, as an all-reduce that writes its result
// before a separate norm kernel would have it (compile-time: on the latency-
// bound row path even a select per element costs time).
template <typename IO, int W, int PPL, int MODE, bool QUANT, bool RES, bool ROUND>
__device__ __forceinline__ void reduce_norm(const RmsParams &p) {
    __shared__ float wave_sums[2][kMaxBlock / 64];
    const int tid = threadIdx.x;
    // launch shape from the arguments and the row length (not from
    // blockDim/gridDim, which go through the dispatch packet in memory)
    const int nthr = lanes_for(p.packs, PPL);
    const int nwaves = nthr >> 6;
    const int64_t stride = p.grid;
    int64_t row = blockIdx.x;    // < T: the launcher never starts more workgroups than rows

    constexpr int NB = W + RES;      // packs loaded per lane pack: partials, residual
    // kSplit: `ahead` receives the next row's loads one row in advance
    u32x4 ahead[PPL][NB];
    if constexpr (MODE == kSplit) load_row<W, PPL, RES, MODE != kRow>(p, row, tid, nthr, ahead);
    // kSplitLeanFew is the kSplitWide body with another store policy
    constexpr bool kWide = MODE == kSplitWide || MODE == kSplitLeanFew;
    // Store policies of residual_out and norm_out, per body, as measured
    // (back-to-back calls, inputs resident in HBM and in the caches):
    //  - looping bodies: both at device scope, norm_out also non-temporal
    //    (1-3 % faster than write-back stores from 2048 rows on, 8192 rows
    //    of eight partials 238.4 -> 233.2 us);
    //  - lean body with at most two rows per workgroup: residual_out at
    //    device scope, norm_out only non-temporal (device scope on norm_out
    //    measured 2-3 % slower there; 1024 rows 32.7 -> 32.55 us);
    //  - row body: residual_out non-temporal (it is next read a layer later;
    //    the FP8 call 4.45 -> 4.02 us), norm_out write-back where the next
    //    layer's GEMM reads it at once, or at device scope with the FP8
    //    epilogue (256 rows of 7168: 4.03 -> 3.69 us; device scope on the
    //    plain row body's stores measured up to 8 % slower on the smallest
    //    calls).
    constexpr int kResidualPolicy = MODE == kRow ? kStoreStream : kStoreDevice;
    constexpr int kNormPolicy = MODE == kRow ? (QUANT ? kStoreDevice : kStorePlain)
                              : MODE == kSplitLeanFew ? kStoreStream
                              : kStoreDeviceStream;
    const uint32_t row_bytes = uint32_t(p.packs) * 16;
    // weight row: loaded once per workgroup and kept in registers.  The
    // split-wide bodies have none to spare: with one pack per lane they keep it
    // in LDS (each lane its own pack, written once), so that nothing after a
    // row's reduction waits on vector memory (a reload from L2 there waited
    // for it and for the row's residual_out stores: measured 1-1.5 % slower);
    // with several packs per lane they reload it per row from L2 after the
    // row's reduction.  Converted where used, so no wait on it stands before
    // the row's loads.
    constexpr bool kWeightLds = kWide && PPL == 1;
    __shared__ u32x4 weight_lds[kWeightLds ? kMaxBlock : 1];
    u32x4 wraw[PPL];
    auto load_weight = [&]() {
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int pk = tid + k * nthr;
            wraw[k] = load16(p.weight + size_t(pk < p.packs ? pk : 0) * 16);
        }
    };
    if constexpr (!kWide || kWeightLds) load_weight();

    // 1/H for the FP8 variant, formed while the row's loads are in flight: its
    // epilogue's dependent chain is long enough that the division after the
    // barrier measured slower (the plain variant divides there: measured faster)
    float inv_h = 1.0f / float(p.H);
    int parity = 0;
    for (;;) {
        u32x4 cur[PPL][NB];
        const int64_t next = row + stride;
        if constexpr (MODE == kSplit) {
#pragma unroll
            for (int k = 0; k < PPL; ++k)
#pragma unroll
                for (int r = 0; r < NB; ++r) cur[k][r] = ahead[k][r];
            if (next < p.T) load_row<W, PPL, RES, MODE != kRow>(p, next, tid, nthr, ahead);
        } else {
            load_row<W, PPL, RES, MODE != kRow>(p, row, tid, nthr, cur);
        }
        // the first row's loads are out: the weight pack (loaded before them)
        // goes to LDS
        if constexpr (kWeightLds)
            if (row == int64_t(blockIdx.x)) weight_lds[tid] = wraw[0];
        // keeps the compiler from moving the division next to its use
        if constexpr (QUANT) asm volatile("" : "+v"(inv_h));
        const size_t base = size_t(row) * size_t(p.H) * 2;

        // phase 1: rank-ordered fp32 sum, residual last, residual_out
        float acc[PPL][8];
        float ss = 0.0f;
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int pk = tid + k * nthr;
            unpack8<IO>(cur[k][0], acc[k]);
#pragma unroll
            for (int r = 1; r < W; ++r) {
                float x[8];
                unpack8<IO>(cur[k][r], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[k][i] = acc[k][i] + x[i];
            }
            if constexpr (ROUND) unpack8<IO>(pack8<IO>(acc[k]), acc[k]);
            if constexpr (RES) {
                float x[8];
                unpack8<IO>(cur[k][W], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[k][i] = acc[k][i] + x[i];
            }
            if constexpr (QUANT) {
                // The FP8 variant adds the row's squares before it packs and
                // stores residual_out (measured 2-4 % faster on its shapes; the
                // plain variant measured faster with the store first).
                if (pk >= p.packs) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[k][i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(acc[k][i], acc[k][i], ss);
                if (pk < p.packs && p.residual_out)
                    store16_policy<kResidualPolicy>(p.residual_out + base, uint32_t(pk) * 16,
                                                    row_bytes, pack8<IO>(acc[k]));
            } else {
                if (pk < p.packs) {
                    if (p.residual_out)
                        store16_policy<kResidualPolicy>(p.residual_out + base, uint32_t(pk) * 16,
                                                        row_bytes, pack8<IO>(acc[k]));
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) acc[k][i] = 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 8; ++i) ss = __builtin_fmaf(acc[k][i], acc[k][i], ss);
            }
        }

        // sum of squares over the row: wave64 reduce, then across wavefronts
        const float wsum = wave_sum(ss);
        if ((tid & 63) == 0) wave_sums[parity][tid >> 6] = wsum;
        __syncthreads();
        float total = 0.0f;
        if constexpr (PPL == 1) {
            total = sum_wave_partials(wave_sums[parity], nwaves, tid);
        } else {
            // rows of several packs per lane have registers for nothing more
            for (int i = 0; i < nwaves; ++i) total += wave_sums[parity][i];
        }
        const float rstd = rsqrtf((QUANT ? total * inv_h : total / float(p.H)) + p.eps);

        // phase 2: normalise, weight, store; optional FP8 group epilogue
        if constexpr (kWeightLds) wraw[0] = weight_lds[tid];
        else if constexpr (kWide) load_weight();
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int pk = tid + k * nthr;
            const bool valid = pk < p.packs;
            float w[8];
            unpack8<IO>(wraw[k], w);
            if (p.options & kGemma) {
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = w[i] + 1.0f;
            }
            float y[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) y[i] = (acc[k][i] * rstd) * w[i];
            if (valid && p.norm_out)
                store16_policy<kNormPolicy>(p.norm_out + base, uint32_t(pk) * 16, row_bytes,
                                            pack8<IO>(y));
            if constexpr (QUANT) {
                float amax = 0.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
                amax = group_max(amax, p.group_lanes);
                const float scale = div448(amax);
                uint32_t lo = 0, hi = 0;
                if (scale != 0.0f) {
                    // The hardware reciprocal (v_rcp_f32, within 1 ulp), then
                    // products: y * inv is within two fp32 roundings of y / scale,
                    // so a code can move one step at a rounding boundary.  Since
                    // |y| <= amax, every quotient is at most 448 * (1 + 2^-22) and
                    // rounds to at most 448: no saturation step is needed.  A scale
                    // below about 2^-128 has no finite reciprocal; those groups
                    // divide.
                    const float inv = __builtin_amdgcn_rcpf(scale);
                    if (__builtin_expect(inv <= 3.40282347e38f, 1)) {
                        lo = pack4_e4m3(y[0] * inv, y[1] * inv, y[2] * inv, y[3] * inv);
                        hi = pack4_e4m3(y[4] * inv, y[5] * inv, y[6] * inv, y[7] * inv);
                    } else {
                        lo = pack4_e4m3(y[0] / scale, y[1] / scale, y[2] / scale, y[3] / scale);
                        hi = pack4_e4m3(y[4] / scale, y[5] / scale, y[6] / scale, y[7] / scale);
                    }
                }
                if (valid) {
                    *reinterpret_cast<u32x2 *>(p.q_out + size_t(row) * p.H + size_t(pk) * 8) =
                        u32x2{lo, hi};
                    // group_lanes is a power of two: the group index is a shift
                    if ((pk & (p.group_lanes - 1)) == 0)
                        p.scales[size_t(row) * p.groups + (pk >> __builtin_ctz(p.group_lanes))] =
                            scale;
                }
            }
        }

        if (MODE == kRow || next >= p.T) break;
        row = next;
        parity ^= 1;
    }
}

// Kernel entry with flat arguments: the first eight (14 dwords: residual,
// weight, H, options and the first four partials) are preloaded into SGPRs at
// wave launch (built with kernarg preloading), so a row's loads start without
// a round trip for their addresses.
template <typename IO, int W, int PPL, int MODE, bool QUANT, bool RES, bool ROUND>
__global__ __launch_bounds__(rms_block_bound(PPL)) void reduce_norm_kernel(
    const uint8_t *residual, const uint8_t *weight, int32_t H, int32_t options,
    const uint8_t *p0, const uint8_t *p1, const uint8_t *p2, const uint8_t *p3,
    const uint8_t *p4, const uint8_t *p5, const uint8_t *p6, const uint8_t *p7,
    uint8_t *norm_out, uint8_t *residual_out, uint8_t *q_out, float *scales, int64_t T,
    float eps, int32_t group_lanes, int32_t grid,
    const uint8_t *p8, const uint8_t *p9, const uint8_t *p10, const uint8_t *p11,
    const uint8_t *p12, const uint8_t *p13, const uint8_t *p14, const uint8_t *p15) {
    RmsParams p;
    p.partials[0] = p0; p.partials[1] = p1; p.partials[2] = p2; p.partials[3] = p3;
    p.partials[4] = p4; p.partials[5] = p5; p.partials[6] = p6; p.partials[7] = p7;
    p.partials[8] = p8; p.partials[9] = p9; p.partials[10] = p10; p.partials[11] = p11;
    p.partials[12] = p12; p.partials[13] = p13; p.partials[14] = p14; p.partials[15] = p15;
    p.residual = residual;
    p.weight = weight;
    p.norm_out = norm_out;
    p.residual_out = residual_out;
    p.q_out = q_out;
    p.scales = scales;
    p.T = T;
    p.H = H;
    p.packs = H >> 3;
    p.eps = eps;
    p.options = options;
    p.group_lanes = group_lanes;
    p.groups = QUANT ? H / (group_lanes * kPackElems) : 0;
    p.grid = grid;
    reduce_norm<IO, W, PPL, MODE, QUANT, RES, ROUND>(p);
}

// ------------------------------------------------------------- QK-norm
// Shard r's base pointer, chosen by selects on values held in registers.
struct Shards {
    const uint8_t *x0, *x1, *x2, *x3, *x4, *x5, *x6, *x7;
    template <int W>
    __device__ __forceinline__ const uint8_t *pick(int r) const {
        const uintptr_t a[kMaxQkW] = {uintptr_t(x0), uintptr_t(x1), uintptr_t(x2), uintptr_t(x3),
                                      uintptr_t(x4), uintptr_t(x5), uintptr_t(x6), uintptr_t(x7)};
        uintptr_t q = a[0];
#pragma unroll
        for (int i = 1; i < W; ++i) q = r == i ? a[i] : q;
        return reinterpret_cast<const uint8_t *>(q);
    }
};

// One workgroup per token.  Each lane adds the squares of its q or k pack to
// the q or the k statistic, and both statistics are reduced across the
// workgroup together.  Element j of shard r's q (or k) part is column
// r * size + j of the concatenated weight.
// LOOP: workgroups loop over tokens (more tokens than workgroups); without it
// every workgroup handles exactly one token in straight-line code.
// ALIGNED: each shard owns lanes_for(q + kv packs, PPL) lanes, a whole number
// of wavefronts, so a wavefront's shard and base pointer are wave-uniform and
// worked out in scalar registers; otherwise (shapes that do not fit 1024 lanes
// that way) the packs are laid out back to back: all shards' q packs, then all
// their k packs, and each lane finds its shard by vector comparisons.
template <typename IO, int W, int PPL, bool LOOP, bool ALIGNED>
__device__ __forceinline__ void qknorm(const QkParams &p, const Shards shards) {
    __shared__ float wave_sums[2][2][kMaxBlock / 64];
    const int tid = threadIdx.x;
    const int per_shard = p.q_packs + p.kv_packs;
    const int nq = W * p.q_packs;
    const int n = nq + W * p.kv_packs;
    const int shard_lanes = lanes_for(per_shard, PPL);
    // launch width (see reduce_norm)
    const int nthr = ALIGNED ? W * shard_lanes : lanes_for(n, PPL);
    const int nwaves = nthr >> 6;
    const size_t row_bytes = size_t(p.q_packs + 2 * p.kv_packs) * 16;
    const int q_size = p.q_packs * 8;
    const int kv_size = p.kv_packs * 8;

    // Row-independent lane layout, worked out once: each pack's shard (by
    // comparisons, no integer division) and its column in the shard row.
    // Aligned: the shard r_al is wave-uniform and `part` is the column within
    // the shard's q or k part; the weight and output addresses are each a
    // choice between two whole q and k address expressions (a product with a
    // per-lane q-or-k factor would be a vector multiply).  Packed: the weight
    // pack and the output offset per lane.  A lane past the end takes pack 0's
    // layout (every address in bounds) and is masked by `valid`.
    bool valid[PPL], is_q[PPL];
    const uint8_t *src[PPL];
    int col[PPL], part[PPL], widx[PPL];
    size_t out_off[PPL];
    int r_al = 0;
    if constexpr (ALIGNED) {
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int shard_waves = shard_lanes >> 6;
        int r = 0;
#pragma unroll
        for (int i = 1; i < W; ++i) r += wave >= i * shard_waves ? 1 : 0;
        const uint8_t *base = shards.pick<W>(r);
        const int lane = tid - r * shard_lanes;
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            const int c0 = lane + k * shard_lanes;   // column pack in the [q | k] row
            valid[k] = c0 < per_shard;
            const int c = valid[k] ? c0 : 0;
            is_q[k] = c < p.q_packs;
            col[k] = c;
            part[k] = is_q[k] ? c : c - p.q_packs;
            src[k] = base;
        }
        r_al = r;
    } else {
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            valid[k] = tid + k * nthr < n;
            const int pk = valid[k] ? tid + k * nthr : 0;
            is_q[k] = pk < nq;
            const int idx = is_q[k] ? pk : pk - nq;
            const int per = is_q[k] ? p.q_packs : p.kv_packs;
            int r = 0;
#pragma unroll
            for (int i = 1; i < W; ++i) r += idx >= i * per ? 1 : 0;
            const int j = idx - r * per;
            widx[k] = idx;
            col[k] = j + (is_q[k] ? 0 : p.q_packs);
            src[k] = shards.pick<W>(r);
            out_off[k] = size_t(r) * size_t(p.T) * size_t(is_q[k] ? q_size : kv_size) * 2 +
                         size_t(j) * 16;
        }
    }

    int64_t row = blockIdx.x;     // < T: the launcher never starts more workgroups than rows
    // Every lane loads (lanes past the end at the clamped pack 0 of shard 0,
    // then zeroed): with no branch around a load, no wait is placed at a join.
    u32x4 xr[PPL], wr[PPL];
#pragma unroll
    for (int k = 0; k < PPL; ++k)
        xr[k] = load16_stream(src[k] + size_t(row) * row_bytes + size_t(col[k]) * 16);
    // weights: loaded once (the same for every token), after the first loads
#pragma unroll
    for (int k = 0; k < PPL; ++k)
        if constexpr (ALIGNED)
            wr[k] = load16(is_q[k] ? p.q_weight + size_t(r_al * p.q_packs + part[k]) * 16
                                   : p.k_weight + size_t(r_al * p.kv_packs + part[k]) * 16);
        else
            wr[k] = load16((is_q[k] ? p.q_weight : p.k_weight) + size_t(widx[k]) * 16);

    int parity = 0;
    for (;;) {
        float x[PPL][8];
        float ssq = 0.0f, ssk = 0.0f;
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            if (!valid[k]) xr[k] = u32x4{0u, 0u, 0u, 0u};
            unpack8<IO>(xr[k], x[k]);
            float s = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) s = __builtin_fmaf(x[k][i], x[k][i], s);
            if (is_q[k]) ssq += s; else ssk += s;
        }
        const int64_t next = row + p.grid;
        if (LOOP && next < p.T) {
#pragma unroll
            for (int k = 0; k < PPL; ++k)
                xr[k] = load16_stream(src[k] + size_t(next) * row_bytes + size_t(col[k]) * 16);
        }
        const float wq = wave_sum(ssq);
        const float wk = wave_sum(ssk);
        if ((tid & 63) == 0) {
            wave_sums[parity][0][tid >> 6] = wq;
            wave_sums[parity][1][tid >> 6] = wk;
        }
        __syncthreads();
        const f32x2 t = sum_wave_partials2(wave_sums[parity][0], wave_sums[parity][1], nwaves, tid);
        const float rq = rsqrtf(t.x / float(W * q_size) + p.eps);
        const float rk = rsqrtf(t.y / float(W * kv_size) + p.eps);
#pragma unroll
        for (int k = 0; k < PPL; ++k) {
            if (valid[k]) {
                float wv[8];
                unpack8<IO>(wr[k], wv);
                const float rs = is_q[k] ? rq : rk;
                float y[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = (x[k][i] * rs) * wv[i];
                // q_out [W, T, q_size], k_out [W, T, kv_size]
                uint8_t *dst;
                if constexpr (ALIGNED) {
                    const size_t out_row = size_t(r_al) * size_t(p.T) + size_t(row);
                    dst = is_q[k] ? p.q_out + (out_row * p.q_packs + part[k]) * 16
                                  : p.k_out + (out_row * p.kv_packs + part[k]) * 16;
                } else {
                    const size_t row_off = size_t(row) * size_t(is_q[k] ? q_size : kv_size) * 2;
                    dst = (is_q[k] ? p.q_out : p.k_out) + out_off[k] + row_off;
                }
                store16(dst, pack8<IO>(y));
            }
        }
        if (!LOOP || next >= p.T) break;
        row = next;
        parity ^= 1;
    }
}

// Kernel entry with flat arguments; the first eight (14 dwords: the sizes, the
// first four shards and both weights) are preloaded into SGPRs at wave launch,
// so every load of a token is issued without waiting for an address.
template <typename IO, int W, int PPL, bool LOOP, bool ALIGNED>
__global__ __launch_bounds__(kMaxBlock) void qknorm_kernel(
    int32_t q_packs, int32_t kv_packs, const uint8_t *x0, const uint8_t *x1, const uint8_t *x2,
    const uint8_t *x3, const uint8_t *q_weight, const uint8_t *k_weight, const uint8_t *x4,
    const uint8_t *x5, const uint8_t *x6, const uint8_t *x7, uint8_t *q_out, uint8_t *k_out,
    int64_t T, float eps, int32_t grid) {
    QkParams p;
    p.x0 = x0; p.x1 = x1; p.x2 = x2; p.x3 = x3;
    p.x4 = x4; p.x5 = x5; p.x6 = x6; p.x7 = x7;
    const Shards shards{x0, x1, x2, x3, x4, x5, x6, x7};
    p.q_weight = q_weight;
    p.k_weight = k_weight;
    p.q_out = q_out;
    p.k_out = k_out;
    p.T = T;
    p.q_packs = q_packs;
    p.kv_packs = kv_packs;
    p.eps = eps;
    p.grid = grid;
    qknorm<IO, W, PPL, LOOP, ALIGNED>(p, shards);
}

// ------------------------------------------------------------- launchers
template <typename IO, int W, int PPL, int MODE, bool QUANT, bool RES, bool ROUND>
hipError_t launch_rms(const RmsParams &p, unsigned grid, unsigned block, hipStream_t s) {
    if (int(block) != lanes_for(p.packs, PPL)) return hipErrorInvalidConfiguration;
    RmsParams a = p;
    a.grid = int32_t(grid);
    void *args[] = {&a.residual, &a.weight, &a.H, &a.options,
                    &a.partials[0], &a.partials[1], &a.partials[2], &a.partials[3],
                    &a.partials[4], &a.partials[5], &a.partials[6], &a.partials[7],
                    &a.norm_out, &a.residual_out, &a.q_out, &a.scales, &a.T, &a.eps,
                    &a.group_lanes, &a.grid,
                    &a.partials[8], &a.partials[9], &a.partials[10], &a.partials[11],
                    &a.partials[12], &a.partials[13], &a.partials[14], &a.partials[15]};
    return hipLaunchKernel(
        reinterpret_cast<const void *>(&reduce_norm_kernel<IO, W, PPL, MODE, QUANT, RES, ROUND>),
        dim3(grid), dim3(block), args, 0, s);
}

template <typename IO, int W, int PPL, bool LOOP, bool ALIGNED>
hipError_t launch_qk(const QkParams &p, unsigned grid, unsigned block, hipStream_t s) {
    const int per_shard = p.q_packs + p.kv_packs;
    const int lanes = ALIGNED ? W * lanes_for(per_shard, PPL) : lanes_for(W * per_shard, PPL);
    if (int(block) != lanes) return hipErrorInvalidConfiguration;
    QkParams a = p;
    a.grid = int32_t(grid);
    void *args[] = {&a.q_packs, &a.kv_packs, &a.x0, &a.x1, &a.x2, &a.x3,
                    &a.q_weight, &a.k_weight, &a.x4, &a.x5, &a.x6, &a.x7,
                    &a.q_out, &a.k_out, &a.T, &a.eps, &a.grid};
    return hipLaunchKernel(reinterpret_cast<const void *>(&qknorm_kernel<IO, W, PPL, LOOP, ALIGNED>),
                           dim3(grid), dim3(block), args, 0, s);
}

template <typename IO, int W, int PPL, int MODE, bool QUANT, bool RES, bool ROUND>
Variant variant() {
    return Variant{
        &launch_rms<IO, W, PPL, MODE, QUANT, RES, ROUND>,
        reinterpret_cast<const void *>(&reduce_norm_kernel<IO, W, PPL, MODE, QUANT, RES, ROUND>)};
}

// Modes built: kRow and kSplit with one pack per lane, kSplitWide with four
// packs per lane (rows longer than 8192 elements), kSplitLean (the kSplitWide
// body with one pack per lane) and kSplitLeanFew (the same with the store
// policy for at most two rows per workgroup) for four to eight partials
// without the FP8 epilogue.
template <typename IO, int W, bool QUANT, bool RES, bool ROUND>
Variant pick_mode(int mode) {
    switch (mode) {
    case kRow: return variant<IO, W, 1, kRow, QUANT, RES, ROUND>();
    case kSplit: return variant<IO, W, 1, kSplit, QUANT, RES, ROUND>();
    case kSplitWide: return variant<IO, W, kMaxPpl, kSplitWide, QUANT, RES, ROUND>();
    case kSplitLean:
        if constexpr (!QUANT && W >= 4) return variant<IO, W, 1, kSplitWide, QUANT, RES, ROUND>();
        return Variant{nullptr, nullptr};
    case kSplitLeanFew:
        if constexpr (!QUANT && W >= 4)
            return variant<IO, W, 1, kSplitLeanFew, QUANT, RES, ROUND>();
        return Variant{nullptr, nullptr};
    default: return Variant{nullptr, nullptr};
    }
}

// More than eight partials: only the persistent body without prefetch, one
// pack per lane (the plan limits such rows to 8192 elements).
template <typename IO, int W, bool QUANT, bool RES, bool ROUND>
Variant pick_mode_many(int mode) {
    if (mode != kSplitWide) return Variant{nullptr, nullptr};
    return variant<IO, W, 1, kSplitWide, QUANT, RES, ROUND>();
}

// W = 1 has no ROUND variant: a single partial is already in the I/O format,
// so rounding the "sum" changes nothing.
template <typename IO, bool QUANT, bool RES, bool ROUND>
Variant pick_w(int W, int mode) {
    switch (W) {
    case 1: return pick_mode<IO, 1, QUANT, RES, false>(mode);
    case 2: return pick_mode<IO, 2, QUANT, RES, ROUND>(mode);
    case 3: return pick_mode<IO, 3, QUANT, RES, ROUND>(mode);
    case 4: return pick_mode<IO, 4, QUANT, RES, ROUND>(mode);
    case 5: return pick_mode<IO, 5, QUANT, RES, ROUND>(mode);
    case 6: return pick_mode<IO, 6, QUANT, RES, ROUND>(mode);
    case 7: return pick_mode<IO, 7, QUANT, RES, ROUND>(mode);
    case 8: return pick_mode<IO, 8, QUANT, RES, ROUND>(mode);
    case 9: return pick_mode_many<IO, 9, QUANT, RES, ROUND>(mode);
    case 10: return pick_mode_many<IO, 10, QUANT, RES, ROUND>(mode);
    case 11: return pick_mode_many<IO, 11, QUANT, RES, ROUND>(mode);
    case 12: return pick_mode_many<IO, 12, QUANT, RES, ROUND>(mode);
    case 13: return pick_mode_many<IO, 13, QUANT, RES, ROUND>(mode);
    case 14: return pick_mode_many<IO, 14, QUANT, RES, ROUND>(mode);
    case 15: return pick_mode_many<IO, 15, QUANT, RES, ROUND>(mode);
    case 16: return pick_mode_many<IO, 16, QUANT, RES, ROUND>(mode);
    default: return Variant{nullptr, nullptr};
    }
}

// The reduce + RMSNorm variants of one I/O format and epilogue.
template <typename IO, bool QUANT>
Variant pick_rms(int W, int mode, bool res, bool round) {
    if (round)
        return res ? pick_w<IO, QUANT, true, true>(W, mode) : pick_w<IO, QUANT, false, true>(W, mode);
    return res ? pick_w<IO, QUANT, true, false>(W, mode) : pick_w<IO, QUANT, false, false>(W, mode);
}

template <typename IO, int W, bool LOOP, bool ALIGNED>
QkLaunch pick_qk_ppl(int ppl) {
    switch (ppl) {
    case 1: return &launch_qk<IO, W, 1, LOOP, ALIGNED>;
    case 2: return &launch_qk<IO, W, 2, LOOP, ALIGNED>;
    case 4: return &launch_qk<IO, W, 4, LOOP, ALIGNED>;
    default: return nullptr;
    }
}

template <typename IO, bool LOOP, bool ALIGNED>
QkLaunch pick_qk_w(int W, int ppl) {
    switch (W) {
    case 1: return pick_qk_ppl<IO, 1, LOOP, ALIGNED>(ppl);
    case 2: return pick_qk_ppl<IO, 2, LOOP, ALIGNED>(ppl);
    case 3: return pick_qk_ppl<IO, 3, LOOP, ALIGNED>(ppl);
    case 4: return pick_qk_ppl<IO, 4, LOOP, ALIGNED>(ppl);
    case 5: return pick_qk_ppl<IO, 5, LOOP, ALIGNED>(ppl);
    case 6: return pick_qk_ppl<IO, 6, LOOP, ALIGNED>(ppl);
    case 7: return pick_qk_ppl<IO, 7, LOOP, ALIGNED>(ppl);
    case 8: return pick_qk_ppl<IO, 8, LOOP, ALIGNED>(ppl);
    default: return nullptr;
    }
}

template <typename IO>
QkLaunch pick_qk(int W, int ppl, bool loop, bool aligned) {
    if (aligned) return loop ? pick_qk_w<IO, true, true>(W, ppl) : pick_qk_w<IO, false, true>(W, ppl);
    return loop ? pick_qk_w<IO, true, false>(W, ppl) : pick_qk_w<IO, false, false>(W, ppl);
}

}  // namespace
}  // namespace arrms
