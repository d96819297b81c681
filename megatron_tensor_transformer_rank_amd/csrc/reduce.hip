// Local reduction of the ranks' partial sums (stand-in for the all-reduce of
// g's forward and f's backward, "Tensor and sequence parallelism", table of
// f and g) with the output bias added once after the sum ("Tensor
// Parallelism's Communication Boundary", on adding a bias before a
// reduction); its sequence-parallel form, the reduce-scatter that keeps one
// rank's block of token rows and adds the residual branch there, and the
// all-gather that concatenates the blocks ("Tensor and sequence
// parallelism", section "Sequence parallelism"); and the column sums of dY
// that are the bias's gradient.
//
// All are HBM-bound streams of 16-byte chunks.  The partial sums are read
// once, with non-temporal loads, up to four ranks at a time; float32
// accumulation in rank order, then the bias, then the residual, and one
// rounding to bf16.  Up to four ranks: one block per output row with the
// whole row's loads in flight; more ranks: a grid-stride loop with four
// chunks per thread.
#include "common.h"
#include "reduce.h"

namespace tpmlp {

constexpr int RD_THREADS = 256;
constexpr int RD_UNROLL = 4;   // output chunks per thread per iteration
constexpr int RD_BATCH = 4;    // ranks loaded before they are added

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p, int64_t chunk) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + chunk);
}
__device__ __forceinline__ void add8(float (&s)[8], u32x4 v) {
  s[0] += bf16lo(v.x); s[1] += bf16hi(v.x);
  s[2] += bf16lo(v.y); s[3] += bf16hi(v.y);
  s[4] += bf16lo(v.z); s[5] += bf16hi(v.z);
  s[6] += bf16lo(v.w); s[7] += bf16hi(v.w);
}

// out chunk q (0 <= q < n_out) = sum_{r<t} p[r][in_off + q] + bias[q % cols8]
// + residual[q].  Consecutive threads take consecutive chunks.
__global__ void __launch_bounds__(RD_THREADS)
reduce_kernel(PartialPtrs pp, int t, int64_t n_out, int64_t in_off, int cols8, const uint16_t* __restrict__ bias,
              const uint16_t* __restrict__ residual, uint16_t* out) {
  const int64_t step = (int64_t)gridDim.x * RD_THREADS * RD_UNROLL;
  for (int64_t q0 = (int64_t)blockIdx.x * RD_THREADS * RD_UNROLL + threadIdx.x; q0 < n_out; q0 += step) {
    float s[RD_UNROLL][8];
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[u][e] = 0.f;
    for (int r0 = 0; r0 < t; r0 += RD_BATCH) {
      u32x4 v[RD_UNROLL][RD_BATCH];
#pragma unroll
      for (int u = 0; u < RD_UNROLL; ++u) {
        const int64_t q = q0 + u * RD_THREADS;
#pragma unroll
        for (int j = 0; j < RD_BATCH; ++j)
          v[u][j] = (r0 + j < t && q < n_out) ? ld_stream(pp.p[r0 + j], in_off + q) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < RD_UNROLL; ++u)
#pragma unroll
        for (int j = 0; j < RD_BATCH; ++j)
          if (r0 + j < t) add8(s[u], v[u][j]);
    }
#pragma unroll
    for (int u = 0; u < RD_UNROLL; ++u) {
      const int64_t q = q0 + u * RD_THREADS;
      if (q >= n_out) continue;
      if (bias) add8(s[u], reinterpret_cast<const u32x4*>(bias)[q % cols8]);
      if (residual) add8(s[u], ld_stream(residual, q));
      uint4 o;
      o.x = pack_bf16x2(s[u][0], s[u][1]);
      o.y = pack_bf16x2(s[u][2], s[u][3]);
      o.z = pack_bf16x2(s[u][4], s[u][5]);
      o.w = pack_bf16x2(s[u][6], s[u][7]);
      reinterpret_cast<uint4*>(out)[q] = o;
    }
  }
}

// One output row per block (256 threads, J 16-byte chunks per thread, the
// residual and all ranks of a batch in flight at once): the row form of
// reduce_kernel, with the same sum order (ranks in order, then the bias, then
// the residual, one rounding), so the two give the same bits.  Used when all
// t ranks fit one batch: with one round of loads per row it streams faster
// (6.3-6.4 TB/s at 4 x [16384, 8192] against 5.9); with two or more batches
// the grid-stride form is faster.
template <int J>
__global__ void __launch_bounds__(RD_THREADS)
reduce_rows_kernel(PartialPtrs pp, int t, int64_t row0, int cols8, const uint16_t* __restrict__ bias,
                   const uint16_t* __restrict__ residual, uint16_t* out) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t in_base = (row0 + row) * cols8, base = row * cols8;
  float v[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
  u32x4 rv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * RD_THREADS;
    rv[j] = (residual && q < cols8) ? ld_stream(residual, base + q) : u32x4{0u, 0u, 0u, 0u};
  }
  for (int r0 = 0; r0 < t; r0 += RD_BATCH) {
    u32x4 c[J][RD_BATCH];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * RD_THREADS;
#pragma unroll
      for (int b = 0; b < RD_BATCH; ++b)
        c[j][b] = (r0 + b < t && q < cols8) ? ld_stream(pp.p[r0 + b], in_base + q) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < J; ++j)
#pragma unroll
      for (int b = 0; b < RD_BATCH; ++b)
        if (r0 + b < t) add8(v[j], c[j][b]);
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * RD_THREADS;
    if (q >= cols8) continue;
    if (bias) add8(v[j], reinterpret_cast<const u32x4*>(bias)[q]);
    if (residual) add8(v[j], rv[j]);
    uint4 o;
    o.x = pack_bf16x2(v[j][0], v[j][1]);
    o.y = pack_bf16x2(v[j][2], v[j][3]);
    o.z = pack_bf16x2(v[j][4], v[j][5]);
    o.w = pack_bf16x2(v[j][6], v[j][7]);
    reinterpret_cast<uint4*>(out)[base + q] = o;
  }
}

namespace {
int64_t stream_blocks(int64_t n_chunks, int num_cu) {
  int64_t blocks = (n_chunks + RD_THREADS * RD_UNROLL - 1) / (RD_THREADS * RD_UNROLL);
  const int64_t cap = (int64_t)num_cu * 16;
  return blocks > cap ? cap : blocks;
}
}  // namespace

hipError_t reduce_partials_launch(const PartialPtrs& pp, int t, int64_t rows, int64_t cols, int64_t row0,
                                  const uint16_t* bias, const uint16_t* residual, uint16_t* out, int num_cu,
                                  hipStream_t st) {
  const int64_t n_out = rows * (cols / 8);
  if (n_out == 0) return hipSuccess;
  const int cols8 = (int)(cols / 8);
  const int need = (cols8 + RD_THREADS - 1) / RD_THREADS;  // chunks per thread of a row
  if (t <= RD_BATCH && need <= 8 && rows < ((int64_t)1 << 30)) {
    const dim3 g((unsigned)rows), b(RD_THREADS);
#define RR(J) hipLaunchKernelGGL((reduce_rows_kernel<J>), g, b, 0, st, pp, t, row0, cols8, bias, residual, out)
    if (need <= 1) RR(1);
    else if (need <= 2) RR(2);
    else if (need <= 4) RR(4);
    else if (need <= 6) RR(6);
    else RR(8);
#undef RR
    return hipGetLastError();
  }
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)stream_blocks(n_out, num_cu)), dim3(RD_THREADS), 0, st, pp, t,
                     n_out, row0 * (cols / 8), (int)(cols / 8), bias, residual, out);
  return hipGetLastError();
}

// out[s * shard_chunks + i] = shards[s][i]; blockIdx.y selects the shard.
__global__ void __launch_bounds__(RD_THREADS)
gather_kernel(PartialPtrs shards, int64_t shard_chunks, uint16_t* out) {
  const uint16_t* src = shards.p[blockIdx.y];
  u32x4* dst = reinterpret_cast<u32x4*>(out) + (int64_t)blockIdx.y * shard_chunks;
  for (int64_t i = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x; i < shard_chunks;
       i += (int64_t)gridDim.x * RD_THREADS)
    dst[i] = ld_stream(src, i);
}

hipError_t gather_launch(const PartialPtrs& shards, int t, int64_t shard_rows, int64_t cols, uint16_t* out,
                         int num_cu, hipStream_t st) {
  const int64_t chunks = shard_rows * (cols / 8);
  if (chunks == 0) return hipSuccess;
  int64_t bx = (chunks + RD_THREADS - 1) / RD_THREADS;
  const int64_t cap = ((int64_t)num_cu * 16 + t - 1) / t;
  if (bx > cap) bx = cap;
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)bx, (unsigned)t), dim3(RD_THREADS), 0, st, shards, chunks, out);
  return hipGetLastError();
}

// db2[c] = sum_r dY[r][c], deterministic in two passes.  Pass 1: block
// (column strip of 512, row slab) -- each lane owns 8 columns (16-byte loads,
// a wave covers 1 KiB of a row, eight of its rows in flight), the 4 waves
// take interleaved rows, their sums meet in LDS in fixed order and the
// slab's float32 partial row goes to the workspace.  Pass 2: one thread per
// column adds the slab partials in order.
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
    // eight of the wave's rows loaded together, then added in row order
    for (int64_t rb = r0 + w; rb < r1; rb += 4 * 8) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t r = rb + 4 * u;
        v[u] = r < r1 ? *reinterpret_cast<const uint4*>(dY + r * cols + c) : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (rb + 4 * u < r1) {
          a[0] += bf16lo(v[u].x); a[1] += bf16hi(v[u].x);
          a[2] += bf16lo(v[u].y); a[3] += bf16hi(v[u].y);
          a[4] += bf16lo(v[u].z); a[5] += bf16hi(v[u].z);
          a[6] += bf16lo(v[u].w); a[7] += bf16hi(v[u].w);
        }
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
  // eight slabs' loads in flight at a time, added in slab order
  for (int q0 = 0; q0 < slabs; q0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = q0 + u < slabs ? part[(int64_t)(q0 + u) * cols + c] : 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (q0 + u < slabs) s += v[u];
  }
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

// p[0, n) = 0: the gradients that are sums over the rows of an empty batch.
// 16-byte stores for the multiple-of-4 head, single floats for the tail.
__global__ void __launch_bounds__(RD_THREADS) zero_f32_kernel(float* __restrict__ p, int64_t n) {
  const int64_t n4 = n / 4, stride = (int64_t)gridDim.x * RD_THREADS;
  const int64_t i0 = (int64_t)blockIdx.x * RD_THREADS + threadIdx.x;
  for (int64_t i = i0; i < n4; i += stride) reinterpret_cast<float4*>(p)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i0 < n - 4 * n4) p[4 * n4 + i0] = 0.f;
}

hipError_t zero_f32_launch(float* p, int64_t n, int num_cu, hipStream_t st) {
  if (p == nullptr || n <= 0) return hipSuccess;
  int64_t blocks = (n / 4 + RD_THREADS - 1) / RD_THREADS;
  const int64_t cap = (int64_t)num_cu * 16;
  if (blocks > cap) blocks = cap;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(RD_THREADS), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace tpmlp
