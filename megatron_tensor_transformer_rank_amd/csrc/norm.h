// Internal interface of the sequence-parallel LayerNorm kernels (norm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "reduce.h"

namespace tpmlp {

constexpr int64_t LN_MAX_COLS = 16384;  // 256 threads x 8 chunks of 8 columns
constexpr int LN_MAX_SLABS = 64;        // row slabs of the backward's column sums (few rows)
// row slabs of the one-pass backward (many rows): 256-thread blocks up to
// 4096 columns (four per CU), 512-thread blocks over 4096 (one per CU)
constexpr int LN_SLAB_BLOCKS_NARROW = 1024;
constexpr int LN_SLAB_BLOCKS_WIDE = 256;
constexpr int LN_MIN_SLAB_ROWS = 8;     // rows per slab, at least

// y = LayerNorm(x) row by row (gamma, beta bf16 [cols]; beta may be NULL);
// mean / rstd float32 [rows] or both NULL.
hipError_t ln_fwd_launch(const uint16_t* x, int64_t rows, int64_t cols, float eps, const uint16_t* gamma,
                         const uint16_t* beta, uint16_t* y, float* mean, float* rstd, hipStream_t st);

// z = bf16(sum_{k<t} pp.p[k][row0 + i, :] + bias + residual[i, :]) (the
// reduce-scatter of reduce_partials_launch), then y = LayerNorm(z) of the
// stored bf16 z, in one pass.
hipError_t ln_fwd_fused_launch(const PartialPtrs& pp, int t, int64_t rows, int64_t cols, int64_t row0,
                               const uint16_t* bias, const uint16_t* residual, uint16_t* z, float eps,
                               const uint16_t* gamma, const uint16_t* beta, uint16_t* y, float* mean, float* rstd,
                               hipStream_t st);

// dx = LayerNorm backward (+ dres), dgamma / dbeta (dbeta may be NULL) over
// the rows; part holds ln_bwd_workspace_bytes(rows, cols).
size_t ln_bwd_workspace_bytes(int64_t rows, int64_t cols);
hipError_t ln_bwd_launch(const uint16_t* x, const uint16_t* gamma, const float* mean, const float* rstd,
                         const uint16_t* dy, const uint16_t* dres, uint16_t* dx, int64_t rows, int64_t cols,
                         float* dgamma, float* dbeta, float* part, hipStream_t st);

struct GradPtrs {
  const float* p[MAX_T];
};
// out[i] = sum_{k<t} g.p[k][i] in rank order (n % 4 == 0).
hipError_t sum_f32_launch(const GradPtrs& g, int t, int64_t n, float* out, hipStream_t st);

}  // namespace tpmlp
