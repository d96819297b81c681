// Local reduction of the ranks' partial sums (stand-in for the all-reduce of
// g's forward and f's backward, "Tensor and sequence parallelism", table of
// f and g) with the output bias added once after the sum ("Tensor
// Parallelism's Communication Boundary", on adding a bias before a
// reduction), and the column sums of dY that are that bias's gradient.
//
// Both are HBM-bound streams: 16-byte loads, float32 accumulation in rank
// order, one rounding to bf16, grid-stride over 8-element chunks.
#include "common.h"
#include "reduce.h"

namespace tpmlp {

constexpr int RD_THREADS = 256;

__global__ void __launch_bounds__(RD_THREADS)
reduce_partials_kernel(PartialPtrs pp, int t, int64_t n_chunks, int cols8, const uint16_t* __restrict__ bias,
                       uint16_t* out) {
  for (int64_t q = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x; q < n_chunks;
       q += (int64_t)gridDim.x * RD_THREADS) {
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < t; ++r) {
      const uint4 v = reinterpret_cast<const uint4*>(pp.p[r])[q];
      s[0] += bf16lo(v.x); s[1] += bf16hi(v.x);
      s[2] += bf16lo(v.y); s[3] += bf16hi(v.y);
      s[4] += bf16lo(v.z); s[5] += bf16hi(v.z);
      s[6] += bf16lo(v.w); s[7] += bf16hi(v.w);
    }
    if (bias) {
      const uint4 b = reinterpret_cast<const uint4*>(bias)[q % cols8];
      s[0] += bf16lo(b.x); s[1] += bf16hi(b.x);
      s[2] += bf16lo(b.y); s[3] += bf16hi(b.y);
      s[4] += bf16lo(b.z); s[5] += bf16hi(b.z);
      s[6] += bf16lo(b.w); s[7] += bf16hi(b.w);
    }
    uint4 o;
    o.x = pack_bf16x2(s[0], s[1]);
    o.y = pack_bf16x2(s[2], s[3]);
    o.z = pack_bf16x2(s[4], s[5]);
    o.w = pack_bf16x2(s[6], s[7]);
    reinterpret_cast<uint4*>(out)[q] = o;
  }
}

hipError_t reduce_partials_launch(const PartialPtrs& pp, int t, int64_t rows, int64_t cols, const uint16_t* bias,
                                  uint16_t* out, int num_cu, hipStream_t st) {
  const int64_t n_chunks = rows * (cols / 8);
  if (n_chunks == 0) return hipSuccess;
  int64_t blocks = (n_chunks + RD_THREADS - 1) / RD_THREADS;
  const int64_t cap = (int64_t)num_cu * 16;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3((unsigned)blocks), dim3(RD_THREADS), 0, st, pp, t, n_chunks,
                     (int)(cols / 8), bias, out);
  return hipGetLastError();
}

// db2[c] = sum_r dY[r][c], deterministic in two passes.  Pass 1: block
// (column strip of 512, row slab) -- each lane owns 8 columns (16-byte loads,
// a wave covers 1 KiB of a row), the 4 waves take interleaved rows, their sums
// meet in LDS in fixed order and the slab's float32 partial row goes to the
// workspace.  Pass 2: one thread per column adds the slab partials in order.
constexpr int CS_STRIP = 512;

int col_sum_slabs(int64_t rows) {
  int64_t rs = (rows + 255) / 256;
  if (rs < 1) rs = 1;
  if (rs > 64) rs = 64;
  return (int)rs;
}

__global__ void __launch_bounds__(RD_THREADS)
col_sum_pass1(const uint16_t* __restrict__ dY, int64_t rows, int64_t cols, int slabs, float* __restrict__ part) {
  __shared__ float red[4][CS_STRIP];
  const int strips = (int)((cols + CS_STRIP - 1) / CS_STRIP);
  const int strip = blockIdx.x % strips, slab = blockIdx.x / strips;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t rpb = (rows + slabs - 1) / slabs;
  const int64_t r0 = (int64_t)slab * rpb;
  const int64_t r1 = r0 + rpb < rows ? r0 + rpb : rows;
  const int64_t c = (int64_t)strip * CS_STRIP + lane * 8;
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < cols) {
    for (int64_t r = r0 + w; r < r1; r += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(dY + r * cols + c);
      a[0] += bf16lo(v.x); a[1] += bf16hi(v.x);
      a[2] += bf16lo(v.y); a[3] += bf16hi(v.y);
      a[4] += bf16lo(v.z); a[5] += bf16hi(v.z);
      a[6] += bf16lo(v.w); a[7] += bf16hi(v.w);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = a[e];
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int cc = tid * 2 + h;
    const int64_t gc = (int64_t)strip * CS_STRIP + cc;
    if (gc < cols) part[(int64_t)slab * cols + gc] = ((red[0][cc] + red[1][cc]) + red[2][cc]) + red[3][cc];
  }
}

__global__ void __launch_bounds__(RD_THREADS)
col_sum_pass2(const float* __restrict__ part, int slabs, int64_t cols, float* __restrict__ db) {
  const int64_t c = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x;
  if (c >= cols) return;
  float s = 0.f;
  for (int q = 0; q < slabs; ++q) s += part[(int64_t)q * cols + c];
  db[c] = s;
}

size_t col_sum_workspace_bytes(int64_t rows, int64_t cols) {
  return (size_t)col_sum_slabs(rows) * (size_t)cols * sizeof(float);
}

hipError_t col_sum_launch(const uint16_t* dY, int64_t rows, int64_t cols, float* db, float* part, hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const int slabs = col_sum_slabs(rows);
  const int64_t strips = (cols + CS_STRIP - 1) / CS_STRIP;
  hipLaunchKernelGGL(col_sum_pass1, dim3((unsigned)(strips * slabs)), dim3(RD_THREADS), 0, st, dY, rows, cols,
                     slabs, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(col_sum_pass2, dim3((unsigned)((cols + RD_THREADS - 1) / RD_THREADS)), dim3(RD_THREADS), 0, st,
                     part, slabs, cols, db);
  return hipGetLastError();
}

}  // namespace tpmlp
