// Host-side internals of libarrms shared by the plan/validation unit (plain C++,
// no HIP headers: it builds and unit-tests with any host compiler) and the HIP
// launch unit.
#pragma once

#include <cstdint>

#include "../../include/arrms.h"

struct ar_rms_plan_s {
    int W;
    int64_t T;
    int64_t H;
    int dtype;
    uint32_t flags;
    int kernel;     // ARRMS_KERNEL_ROW / ARRMS_KERNEL_SPLIT
    int block;      // threads per workgroup of the reduce+norm kernel
    int ppl;        // 16-byte packs per lane of the reduce+norm kernel
};

namespace arrms {

constexpr int kMaxW = 16;           // partial buffers per reduce+norm call
constexpr int kMaxPrefetchW = 8;    // beyond: no row-ahead prefetch, rows of at most 8192
constexpr int kMaxQkW = 8;          // shards per QK-norm call
constexpr int kPackElems = 8;       // 16-byte pack of 16-bit elements
constexpr int kMaxBlock = 1024;     // threads per workgroup
constexpr int kMaxPpl = 4;          // packs per lane of the reduce+norm kernel (rows > 8192)
constexpr int kMaxQkPpl = 4;        // packs per lane of the QK-norm kernel
constexpr int64_t kMaxRowTokens = 80;
constexpr int64_t kMaxH = int64_t(kMaxBlock / 2) * kMaxPpl * kPackElems;   // 16384

// Records `msg` as the calling thread's last error and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the calling thread's last error (each entry point starts with it).
void clear_error();

// Launch shape of the reduce+norm kernels: threads and packs per lane.
struct Shape {
    int block;
    int ppl;
};
Shape row_shape(int64_t H);
Shape split_shape(int64_t H);
Shape qk_shape(int W, int q_size, int kv_size);
Shape qk_aligned_shape(int W, int q_size, int kv_size);   // {0, 0}: does not fit

// Argument checks of the run entry points; return ARRMS_OK or the status to
// return (with the message recorded).
int check_rms_args(const ar_rms_plan_s *plan, const void *const *partials,
                   const void *residual, const void *weight, float eps,
                   const void *norm_out, bool norm_required, const void *residual_out);
int check_quant_args(const ar_rms_plan_s *plan, int group_size, const void *q_out,
                     const void *scales);
int check_qk_args(const ar_rms_plan_s *plan, const void *const *qkv, int q_size, int kv_size,
                  const void *q_weight, const void *k_weight, float eps, const void *q_out,
                  const void *k_out);

}  // namespace arrms
