// Internal interface of the reduction kernels (reduce.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

constexpr int MAX_T = 64;

struct PartialPtrs {
  const uint16_t* p[MAX_T];
};

// out [rows, cols] = sum_{r<t} pp.p[r][row0 + i, :] (rank order, float32)
// + bias (once, may be NULL) + residual[i, :] (may be NULL), one rounding.
hipError_t reduce_partials_launch(const PartialPtrs& pp, int t, int64_t rows, int64_t cols, int64_t row0,
                                  const uint16_t* bias, const uint16_t* residual, uint16_t* out, int num_cu,
                                  hipStream_t st);
// out [t * shard_rows, cols] = the t shards [shard_rows, cols] stacked in order.
hipError_t gather_launch(const PartialPtrs& shards, int t, int64_t shard_rows, int64_t cols, uint16_t* out,
                         int num_cu, hipStream_t st);
// db2 = column sums of dY; part is col_sum_workspace_bytes(rows, cols) of
// device scratch.
size_t col_sum_workspace_bytes(int64_t rows, int64_t cols);
hipError_t col_sum_launch(const uint16_t* dY, int64_t rows, int64_t cols, float* db, float* part, hipStream_t st);
// p[0, n) = 0 (p 16-byte aligned; NULL or n <= 0: nothing is launched).
hipError_t zero_f32_launch(float* p, int64_t n, int num_cu, hipStream_t st);

}  // namespace tpmlp
