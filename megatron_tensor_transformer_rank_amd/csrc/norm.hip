// LayerNorm of the sequence-parallel region for gfx950: forward (optionally
// fused with the reduce-scatter that leaves the tensor-parallel region, its
// output bias and the residual addition), backward (with the residual
// branch's gradient added), and the sum over ranks of the LayerNorm weight's
// gradient ("Tensor and sequence parallelism", section "Sequence
// parallelism": the LayerNorms, dropouts and residual additions work on the
// rank's s/t token rows, and the weights shared by those blocks need their
// gradients summed over the group).
//
// All HBM-bound streams of 16-byte chunks.  A block owns a whole row
// (LayerNorm needs the row's statistics), 256 threads, or 1024 when there are
// fewer than 1024 rows: thread i holds chunks i, i + NT, ... of the row in
// registers, so every element is read once and
// the statistics come from registers in two passes (mean, then the biased
// variance of the centred values).  Block sums: a butterfly over the 64 lanes
// (every lane ends with the same bits), then the waves in wave order, so
// results are deterministic.  The fused forward adds the t partial sums in
// float32 in rank order, then the bias, then the residual, rounds z to bf16,
// stores it, and normalises that stored value: bit for bit what a separate
// reduce-scatter followed by a LayerNorm of z computes.
//
// The backward, for many rows (4096 and more), is one pass over row slabs:
// a block per slab (every S-th row, so that the grid sweeps the tensors in
// row order) forms dx row by row and keeps its columns' dgamma / dbeta sums
// in registers, then a kernel adds the slabs' partial rows in slab order.  For fewer rows it runs as column tiles, dgamma and dbeta over
// (512-column strip, row slab) tiles with at most 64 slabs of partial rows,
// beside the row kernel (dx, one row per block, like the forward) in the same
// launch, then the slab sums; when dx overwrites dy in place the column
// kernel, the slab sums and the row kernel run one after another.  The
// column tiles re-read x and dy but keep every CU busy where one block per
// slab would leave most of them idle.
#include "common.h"
#include "norm.h"

namespace tpmlp {

constexpr int LN_THREADS = 256;
constexpr int LN_WAVES = LN_THREADS / 64;
constexpr int LN_BATCH = 4;  // ranks loaded before they are added
constexpr int SS_GROUPS = 16;
constexpr int SS_BATCH = 8;  // slab loads in flight per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ u32x4 ld_nt(const uint16_t* p, int64_t chunk) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + chunk);
}
__device__ __forceinline__ u32x4 ld_c(const uint16_t* p, int64_t chunk) {
  return reinterpret_cast<const u32x4*>(p)[chunk];
}
__device__ __forceinline__ void unpack8(u32x4 v, float (&f)[8]) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x);
  f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z);
  f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}
__device__ __forceinline__ void add8(float (&s)[8], u32x4 v) {
  s[0] += bf16lo(v.x); s[1] += bf16hi(v.x);
  s[2] += bf16lo(v.y); s[3] += bf16hi(v.y);
  s[4] += bf16lo(v.z); s[5] += bf16hi(v.z);
  s[6] += bf16lo(v.w); s[7] += bf16hi(v.w);
}
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Sum of v over a block of NW waves; red is NW floats of LDS used by this
// call only.  Every thread returns the same value.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) s += red[w];
  return s;
}

// Two block sums with one barrier: red is [2][NW] floats of LDS; the caller
// alternates `slot` (0, 1, 0, ...) between consecutive calls, so a fast wave
// writing the next call's values never meets a slow wave still reading this
// call's.  Every thread returns the same two values.
template <int NW>
__device__ __forceinline__ void block_sum2(float& a, float& b, float (*red)[2][NW], int slot) {
  a = wave_sum(a);
  b = wave_sum(b);
  if ((threadIdx.x & 63) == 0) {
    red[slot][0][threadIdx.x >> 6] = a;
    red[slot][1][threadIdx.x >> 6] = b;
  }
  __syncthreads();
  a = red[slot][0][0];
  b = red[slot][1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    a += red[slot][0][w];
    b += red[slot][1][w];
  }
}

}  // namespace

// One row per block of NT threads.  FUSED: the row is row0 + blockIdx.x of
// the partial sums (plus bias and residual), stored to z; otherwise it is row
// blockIdx.x of x.
template <int NT, int J, bool FUSED>
__global__ void __launch_bounds__(NT)
ln_fwd_kernel(PartialPtrs pp, int t, int64_t row0, const uint16_t* __restrict__ bias, const uint16_t* residual,
              uint16_t* z, const uint16_t* x, int cols8, int cols, float eps, const uint16_t* __restrict__ gamma,
              const uint16_t* __restrict__ beta, uint16_t* y, float* __restrict__ mean_out,
              float* __restrict__ rstd_out) {
  __shared__ float red[2][NT / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t base = row * cols8;
  float v[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[j][e] = 0.f;

  if constexpr (FUSED) {
    const int64_t in_base = (row0 + row) * cols8;
    // the residual is loaded with the first batch of partials
    u32x4 rv[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * NT;
      rv[j] = (residual && q < cols8) ? ld_nt(residual, base + q) : u32x4{0u, 0u, 0u, 0u};
    }
    for (int r0 = 0; r0 < t; r0 += LN_BATCH) {
      u32x4 c[J][LN_BATCH];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int q = tid + j * NT;
#pragma unroll
        for (int b = 0; b < LN_BATCH; ++b)
          c[j][b] = (r0 + b < t && q < cols8) ? ld_nt(pp.p[r0 + b], in_base + q) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int b = 0; b < LN_BATCH; ++b)
          if (r0 + b < t) add8(v[j], c[j][b]);
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * NT;
      if (q < cols8) {
        if (bias) add8(v[j], ld_c(bias, q));
        if (residual) add8(v[j], rv[j]);
        const u32x4 o = pack8(v[j]);
        reinterpret_cast<u32x4*>(z)[base + q] = o;
        unpack8(o, v[j]);  // the LayerNorm reads z as stored
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] = 0.f;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * NT;
      if (q < cols8) unpack8(ld_nt(x, base + q), v[j]);
    }
  }

  float s = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) s += v[j][e];
  const float mean = block_sum<NT / 64>(s, red[0]) / (float)cols;
  float d = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (tid + j * NT < cols8) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = v[j][e] - mean;
        d += c * c;
      }
    }
  }
  const float var = block_sum<NT / 64>(d, red[1]) / (float)cols;
  const float rstd = 1.0f / sqrtf(var + eps);

#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * NT;
    if (q < cols8) {
      float g[8], b[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, o[8];
      unpack8(ld_c(gamma, q), g);
      if (beta) unpack8(ld_c(beta, q), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[j][e] - mean) * rstd * g[e] + b[e];
      reinterpret_cast<u32x4*>(y)[base + q] = pack8(o);
    }
  }
  if (tid == 0 && mean_out) {
    mean_out[row] = mean;
    rstd_out[row] = rstd;
  }
}

// One row per block of NT threads: xhat = (x - mean) * rstd, g = dy * gamma,
// dx = rstd * (g - sum(g)/h - xhat * sum(g * xhat)/h) (+ dres).  red: the
// block's [2][NT/64] floats of LDS.
template <int NT, int J>
__device__ __forceinline__ void ln_dx_row(int64_t r, const uint16_t* x, const uint16_t* __restrict__ gamma,
                                          const float* __restrict__ mean, const float* __restrict__ rstd,
                                          const uint16_t* dy, const uint16_t* dres, uint16_t* dx, int cols8, int cols,
                                          float (*red)[NT / 64]) {
  const int tid = threadIdx.x;
  const int64_t base = r * cols8;
  const float mu = mean[r], rs = rstd[r];
  // dres is loaded with x and dy: one round trip to memory per row
  u32x4 xv[J], dv[J], rv[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * NT;
    xv[j] = q < cols8 ? ld_nt(x, base + q) : u32x4{0u, 0u, 0u, 0u};
    dv[j] = q < cols8 ? ld_nt(dy, base + q) : u32x4{0u, 0u, 0u, 0u};
    rv[j] = (dres && q < cols8) ? ld_nt(dres, base + q) : u32x4{0u, 0u, 0u, 0u};
  }
  float s1 = 0.f, s2 = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * NT;
    if (q < cols8) {
      float xf[8], df[8], gm[8];
      unpack8(xv[j], xf);
      unpack8(dv[j], df);
      unpack8(ld_c(gamma, q), gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = df[e] * gm[e];
        s1 += g;
        s2 += g * ((xf[e] - mu) * rs);
      }
    }
  }
  const float m1 = block_sum<NT / 64>(s1, red[0]) / (float)cols;
  const float m2 = block_sum<NT / 64>(s2, red[1]) / (float)cols;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * NT;
    if (q < cols8) {
      float xf[8], df[8], gm[8], o[8];
      unpack8(xv[j], xf);
      unpack8(dv[j], df);
      unpack8(ld_c(gamma, q), gm);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rs * (df[e] * gm[e] - m1 - (xf[e] - mu) * rs * m2);
      if (dres) add8(o, rv[j]);
      reinterpret_cast<u32x4*>(dx)[base + q] = pack8(o);
    }
  }
}

template <int NT, int J>
__global__ void __launch_bounds__(NT)
ln_bwd_dx_kernel(const uint16_t* x, const uint16_t* __restrict__ gamma, const float* __restrict__ mean,
                 const float* __restrict__ rstd, const uint16_t* dy, const uint16_t* dres, uint16_t* dx, int cols8,
                 int cols) {
  __shared__ float red[2][NT / 64];
  ln_dx_row<NT, J>(blockIdx.x, x, gamma, mean, rstd, dy, dres, dx, cols8, cols, red);
}

// The backward in one pass (many rows): block b of S takes the rows b,
// b + S, b + 2S, ... one after another, so that at any moment the grid's
// blocks read neighbouring rows and sweep each tensor front to back.  NT
// threads per row (256 up to 4096 columns, 512 over that), thread i holding
// chunks i, i + NT, ... of a row.  Per row it forms dx with the arithmetic of
// ln_dx_row and adds the row's dy * xhat and dy to its columns' dgamma /
// dbeta sums in registers, in row order; the next row's loads are issued
// before this row's sums.  At the end the block writes its partial dgamma /
// dbeta rows, which slab_sum_kernel adds in block order.  dx may coincide
// with dy or dres: a row is read whole before it is written.
template <int NT, int J>
__global__ void __launch_bounds__(NT)
ln_bwd_slab_kernel(const uint16_t* x, const uint16_t* __restrict__ gamma, const float* __restrict__ mean,
                   const float* __restrict__ rstd, const uint16_t* dy, const uint16_t* dres, uint16_t* dx,
                   int64_t rows, int cols8, int cols, float* __restrict__ part_g, float* __restrict__ part_b) {
  __shared__ float red[2][2][NT / 64];
  const int tid = threadIdx.x;
  const int64_t step = gridDim.x;
  float ag[J][8], ab[J][8];
#pragma unroll
  for (int j = 0; j < J; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[j][e] = ab[j][e] = 0.f;
  u32x4 xv[J], dv[J], rv[J];
  auto load = [&](int64_t r, u32x4 (&xa)[J], u32x4 (&da)[J], u32x4 (&ra)[J]) __attribute__((always_inline)) {
    const int64_t base = r * cols8;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * NT;
      const bool ok = r < rows && q < cols8;
      xa[j] = ok ? ld_nt(x, base + q) : u32x4{0u, 0u, 0u, 0u};
      da[j] = ok ? ld_nt(dy, base + q) : u32x4{0u, 0u, 0u, 0u};
      ra[j] = (dres && ok) ? ld_nt(dres, base + q) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // the thread's gamma chunks stay in registers: reloaded per row, their
  // latency (behind the streaming traffic) sat on every row's path
  u32x4 gp[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * NT;
    gp[j] = q < cols8 ? ld_c(gamma, q) : u32x4{0u, 0u, 0u, 0u};
  }
  load(blockIdx.x, xv, dv, rv);
  int slot = 0;
  for (int64_t r = blockIdx.x; r < rows; r += step, slot ^= 1) {
    u32x4 xn[J], dn[J], rn[J];
    load(r + step, xn, dn, rn);  // past the last row: no loads, zeros
    const float mu = mean[r], rs = rstd[r];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * NT;
      if (q < cols8) {
        float xf[8], df[8], gm[8];
        unpack8(xv[j], xf);
        unpack8(dv[j], df);
        unpack8(gp[j], gm);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (xf[e] - mu) * rs;
          const float g = df[e] * gm[e];
          s1 += g;
          s2 += g * xh;
          ag[j][e] += df[e] * xh;
          ab[j][e] += df[e];
        }
      }
    }
    block_sum2<NT / 64>(s1, s2, red, slot);
    const float m1 = s1 / (float)cols, m2 = s2 / (float)cols;
    const int64_t base = r * cols8;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int q = tid + j * NT;
      if (q < cols8) {
        float xf[8], df[8], gm[8], o[8];
        unpack8(xv[j], xf);
        unpack8(dv[j], df);
        unpack8(gp[j], gm);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = rs * (df[e] * gm[e] - m1 - (xf[e] - mu) * rs * m2);
        if (dres) add8(o, rv[j]);
        reinterpret_cast<u32x4*>(dx)[base + q] = pack8(o);
      }
    }
#pragma unroll
    for (int j = 0; j < J; ++j) {
      xv[j] = xn[j];
      dv[j] = dn[j];
      rv[j] = rn[j];
    }
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int q = tid + j * NT;
    if (q < cols8) {
      float* pg = part_g + (int64_t)blockIdx.x * cols + (int64_t)q * 8;
      reinterpret_cast<float4*>(pg)[0] = make_float4(ag[j][0], ag[j][1], ag[j][2], ag[j][3]);
      reinterpret_cast<float4*>(pg)[1] = make_float4(ag[j][4], ag[j][5], ag[j][6], ag[j][7]);
      if (part_b) {
        float* pb = part_b + (int64_t)blockIdx.x * cols + (int64_t)q * 8;
        reinterpret_cast<float4*>(pb)[0] = make_float4(ab[j][0], ab[j][1], ab[j][2], ab[j][3]);
        reinterpret_cast<float4*>(pb)[1] = make_float4(ab[j][4], ab[j][5], ab[j][6], ab[j][7]);
      }
    }
  }
}

// dgamma / dbeta partial rows of one (column strip, row slab) tile: a lane
// owns 8 adjacent columns (16-byte loads, a wave covers 512 columns), the 4
// waves take interleaved rows of the slab, UNROLL rows of loads in flight
// (four; one in the 1024-thread few-row kernel, whose registers are held to
// 64 without spilling so that two blocks share a CU), and their sums meet in
// LDS in wave order.  The rows are added in the same order either way.
constexpr int LN_DG_STRIP = 512;

// The tile's code for one group of LN_THREADS threads (gtid = the thread's
// index in its group; red = the group's [LN_WAVES][LN_DG_STRIP] floats of
// LDS).  Every thread of the block reaches the same barriers: a group whose
// tile is past the last one (live = false) loads and stores nothing.
template <int UNROLL>
__device__ __forceinline__ void ln_dgb_tile(int tile, bool live, int gtid, const uint16_t* __restrict__ x,
                                            const float* __restrict__ mean, const float* __restrict__ rstd,
                                            const uint16_t* __restrict__ dy, int64_t rows, int64_t cols, int64_t rpb,
                                            float* __restrict__ part_g, float* __restrict__ part_b,
                                            float (*red)[LN_DG_STRIP]) {
  const int strips = (int)((cols + LN_DG_STRIP - 1) / LN_DG_STRIP);
  const int strip = tile % strips, slab = tile / strips;
  const int lane = gtid & 63, w = gtid >> 6;
  const int64_t r0 = (int64_t)slab * rpb;
  const int64_t r1 = !live ? r0 : (r0 + rpb < rows ? r0 + rpb : rows);
  const int64_t c = (int64_t)strip * LN_DG_STRIP + lane * 8;
  const bool cok = live && c < cols;
  float ag[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, ab[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int64_t rb = r0 + w; rb < r1; rb += LN_WAVES * UNROLL) {
    u32x4 xv[UNROLL], dv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t r = rb + (int64_t)u * LN_WAVES;
      const bool ok = cok && r < r1;
      xv[u] = ok ? ld_nt(x + r * cols + c, 0) : u32x4{0u, 0u, 0u, 0u};
      dv[u] = ok ? ld_nt(dy + r * cols + c, 0) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int64_t r = rb + (int64_t)u * LN_WAVES;
      if (cok && r < r1) {
        const float mu = mean[r], rs = rstd[r];
        float xf[8], df[8];
        unpack8(xv[u], xf);
        unpack8(dv[u], df);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ag[e] += df[e] * ((xf[e] - mu) * rs);
          ab[e] += df[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = ag[e];
  __syncthreads();
  if (live)
    for (int cc = gtid; cc < LN_DG_STRIP; cc += LN_THREADS) {
      const int64_t gc = (int64_t)strip * LN_DG_STRIP + cc;
      if (gc < cols) part_g[(int64_t)slab * cols + gc] = ((red[0][cc] + red[1][cc]) + red[2][cc]) + red[3][cc];
    }
  if (!part_b) return;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = ab[e];
  __syncthreads();
  if (live)
    for (int cc = gtid; cc < LN_DG_STRIP; cc += LN_THREADS) {
      const int64_t gc = (int64_t)strip * LN_DG_STRIP + cc;
      if (gc < cols) part_b[(int64_t)slab * cols + gc] = ((red[0][cc] + red[1][cc]) + red[2][cc]) + red[3][cc];
    }
}

__global__ void __launch_bounds__(LN_THREADS)
ln_bwd_dgb_kernel(const uint16_t* __restrict__ x, const float* __restrict__ mean, const float* __restrict__ rstd,
                  const uint16_t* __restrict__ dy, int64_t rows, int64_t cols, int64_t rpb,
                  float* __restrict__ part_g, float* __restrict__ part_b) {
  __shared__ float red[LN_WAVES][LN_DG_STRIP];
  ln_dgb_tile<4>(blockIdx.x, true, threadIdx.x, x, mean, rstd, dy, rows, cols, rpb, part_g, part_b, red);
}

// The two independent halves of the few-row backward in one launch, when dx
// does not overwrite dy: blocks [0, ndg) take NT / 256 dgamma / dbeta tiles
// each (one per group of 256 threads, tile = NT / 256 * block + group, the
// arithmetic of ln_bwd_dgb_kernel), blocks [ndg, ndg + rows) one dx row each
// (ln_bwd_dx_kernel's arithmetic).  Same bits as the two kernels.
template <int NT, int J>
__global__ void __launch_bounds__(NT, NT == 1024 ? 8 : 1)
ln_bwd_few_kernel(const uint16_t* x, const uint16_t* __restrict__ gamma, const float* __restrict__ mean,
                  const float* __restrict__ rstd, const uint16_t* dy, const uint16_t* dres, uint16_t* dx, int cols8,
                  int64_t rows, int64_t cols, int64_t rpb, int ntiles, int ndg, float* __restrict__ part_g,
                  float* __restrict__ part_b) {
  constexpr int GROUPS = NT / LN_THREADS;
  __shared__ float red_g[GROUPS][LN_WAVES][LN_DG_STRIP];
  __shared__ float red_x[2][NT / 64];
  if ((int)blockIdx.x < ndg) {
    const int grp = threadIdx.x / LN_THREADS;
    const int tile = (int)blockIdx.x * GROUPS + grp;
    ln_dgb_tile<NT == 1024 ? 1 : 4>(tile, tile < ntiles, threadIdx.x % LN_THREADS, x, mean, rstd, dy, rows, cols,
                                     rpb, part_g, part_b, red_g[grp]);
  } else {
    ln_dx_row<NT, J>((int64_t)blockIdx.x - ndg, x, gamma, mean, rstd, dy, dres, dx, cols8, (int)cols, red_x);
  }
}

// out[c] = sum_{q<slabs} part[q][c], for one or two (part, out) pairs.  A
// block owns 64 columns (16 float4 lanes); its 16 groups each add every 16th
// slab in increasing order, then the group sums are added in group order.
__global__ void __launch_bounds__(LN_THREADS)
slab_sum_kernel(const float* __restrict__ part0, float* __restrict__ out0, const float* __restrict__ part1,
                float* __restrict__ out1, int slabs, int64_t cols) {
  // blockIdx.y: 0 for the first sum, 1 for the second
  const float* part = blockIdx.y ? part1 : part0;
  float* out = blockIdx.y ? out1 : out0;
  __shared__ float4 red[SS_GROUPS][16];
  const int c4 = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const int64_t c = (int64_t)blockIdx.x * 64 + c4 * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < cols) {
    // SS_BATCH loads in flight, then added in increasing slab order
    for (int q0 = grp; q0 < slabs; q0 += SS_GROUPS * SS_BATCH) {
      float4 v[SS_BATCH];
#pragma unroll
      for (int u = 0; u < SS_BATCH; ++u) {
        const int q = q0 + u * SS_GROUPS;
        v[u] = q < slabs ? *reinterpret_cast<const float4*>(part + (int64_t)q * cols + c)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < SS_BATCH; ++u)
        if (q0 + u * SS_GROUPS < slabs) {
          a.x += v[u].x; a.y += v[u].y; a.z += v[u].z; a.w += v[u].w;
        }
    }
  }
  red[grp][c4] = a;
  __syncthreads();
  if (grp == 0 && c < cols) {
    float4 r = red[0][c4];
#pragma unroll
    for (int q = 1; q < SS_GROUPS; ++q) {
      const float4 o = red[q][c4];
      r.x += o.x; r.y += o.y; r.z += o.z; r.w += o.w;
    }
    *reinterpret_cast<float4*>(out + c) = r;
  }
}

// out[i] = sum_{k<t} g.p[k][i], float4 per thread, rank order.
__global__ void __launch_bounds__(LN_THREADS)
sum_f32_kernel(GradPtrs g, int t, int64_t n4, float* __restrict__ out) {
  for (int64_t i = (int64_t)blockIdx.x * LN_THREADS + threadIdx.x; i < n4; i += (int64_t)gridDim.x * LN_THREADS) {
    float4 s = reinterpret_cast<const float4*>(g.p[0])[i];
    for (int k = 1; k < t; ++k) {
      const float4 v = reinterpret_cast<const float4*>(g.p[k])[i];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    reinterpret_cast<float4*>(out)[i] = s;
  }
}

namespace {

// Threads per row: 1024 (16 waves) when there are few rows, so that every
// CU still holds enough loads in flight; 256 otherwise.  A function of the
// row count only, so the fused and the separate forward pick the same.
constexpr int LN_FEW_ROWS = 1024;
constexpr int64_t LN_ONE_PASS_ROWS = 4096;  // measured: below it the two-pass form is as fast or faster
int ln_nt(int64_t rows) { return rows < LN_FEW_ROWS ? 1024 : LN_THREADS; }

// chunks per thread, the smallest instantiated J >= cols8 / nt
int ln_j(int64_t cols, int nt) {
  const int64_t need = (cols / 8 + nt - 1) / nt;
  static const int js[] = {1, 2, 3, 4, 6, 8};
  for (int j : js)
    if (j >= need && (nt == LN_THREADS || j <= 2)) return j;
  return 0;
}

// Many rows: the one-pass backward (ln_bwd_slab_kernel); few rows: the
// column kernel, the slab sums, then the 1024-thread row kernel, which keep
// every CU busy where a slab per block would leave most of them idle.
bool bwd_one_pass(int64_t rows) { return rows >= LN_ONE_PASS_ROWS; }

// Threads per row of the one-pass backward: 256 up to 4096 columns (one or
// two chunks per thread, four blocks per CU), 512 over that (two to four
// chunks, one block per CU).  Measured on 4096 x 8192, 8192 x 8192,
// 16384 x 4096 and 4100 x 12288 against 256 threads with up to four chunks
// and other slab counts.
int bwd_slab_nt(int64_t cols) { return cols / 8 > 2 * LN_THREADS ? 512 : LN_THREADS; }

// Row slabs of the backward's dgamma / dbeta partial sums, at least
// LN_MIN_SLAB_ROWS rows each.  The one-pass kernel: one block per slab, at
// most LN_SLAB_BLOCKS_NARROW 256-thread or LN_SLAB_BLOCKS_WIDE 512-thread
// blocks, the slab being every slabs-th row.  The column kernel: at most
// LN_MAX_SLABS runs of rpb consecutive rows.
void bwd_slabs(int64_t rows, int64_t cols, int& slabs, int64_t& rpb) {
  int64_t nb = (rows + LN_MIN_SLAB_ROWS - 1) / LN_MIN_SLAB_ROWS;
  const int64_t cap = !bwd_one_pass(rows)                   ? LN_MAX_SLABS
                      : bwd_slab_nt(cols) == LN_THREADS ? LN_SLAB_BLOCKS_NARROW
                                                        : LN_SLAB_BLOCKS_WIDE;
  if (nb > cap) nb = cap;
  if (nb < 1) nb = 1;
  rpb = (rows + nb - 1) / nb;
  if (rpb < 1) rpb = 1;
  slabs = bwd_one_pass(rows) ? (int)nb : (int)((rows + rpb - 1) / rpb);
}

template <bool FUSED>
hipError_t fwd_dispatch(const PartialPtrs& pp, int t, int64_t rows, int64_t cols, int64_t row0,
                        const uint16_t* bias, const uint16_t* residual, uint16_t* z, const uint16_t* x, float eps,
                        const uint16_t* gamma, const uint16_t* beta, uint16_t* y, float* mean, float* rstd,
                        hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int cols8 = (int)(cols / 8);
  const int nt = ln_nt(rows);
  const dim3 grid((unsigned)rows), blk(nt);
#define LN_FWD(NT, J)                                                                                          \
  hipLaunchKernelGGL((ln_fwd_kernel<NT, J, FUSED>), grid, blk, 0, st, pp, t, row0, bias, residual, z, x,      \
                     cols8, (int)cols, eps, gamma, beta, y, mean, rstd)
  const int j = ln_j(cols, nt);
  if (nt == 1024) {
    if (j == 1) LN_FWD(1024, 1);
    else if (j == 2) LN_FWD(1024, 2);
    else return hipErrorInvalidValue;
  } else {
    switch (j) {
      case 1: LN_FWD(LN_THREADS, 1); break;
      case 2: LN_FWD(LN_THREADS, 2); break;
      case 3: LN_FWD(LN_THREADS, 3); break;
      case 4: LN_FWD(LN_THREADS, 4); break;
      case 6: LN_FWD(LN_THREADS, 6); break;
      case 8: LN_FWD(LN_THREADS, 8); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef LN_FWD
  return hipGetLastError();
}

}  // namespace

hipError_t ln_fwd_launch(const uint16_t* x, int64_t rows, int64_t cols, float eps, const uint16_t* gamma,
                         const uint16_t* beta, uint16_t* y, float* mean, float* rstd, hipStream_t st) {
  const PartialPtrs none = {};
  return fwd_dispatch<false>(none, 0, rows, cols, 0, nullptr, nullptr, nullptr, x, eps, gamma, beta, y, mean, rstd,
                             st);
}

hipError_t ln_fwd_fused_launch(const PartialPtrs& pp, int t, int64_t rows, int64_t cols, int64_t row0,
                               const uint16_t* bias, const uint16_t* residual, uint16_t* z, float eps,
                               const uint16_t* gamma, const uint16_t* beta, uint16_t* y, float* mean, float* rstd,
                               hipStream_t st) {
  return fwd_dispatch<true>(pp, t, rows, cols, row0, bias, residual, z, nullptr, eps, gamma, beta, y, mean, rstd, st);
}

size_t ln_bwd_workspace_bytes(int64_t rows, int64_t cols) {
  int slabs;
  int64_t rpb;
  bwd_slabs(rows, cols, slabs, rpb);
  return (size_t)2 * (size_t)slabs * (size_t)cols * sizeof(float);
}

hipError_t ln_bwd_launch(const uint16_t* x, const uint16_t* gamma, const float* mean, const float* rstd,
                         const uint16_t* dy, const uint16_t* dres, uint16_t* dx, int64_t rows, int64_t cols,
                         float* dgamma, float* dbeta, float* part, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 blk(LN_THREADS);
  int slabs;
  int64_t rpb;
  bwd_slabs(rows, cols, slabs, rpb);
  float* part_g = part;
  float* part_b = dbeta ? part + (int64_t)slabs * cols : nullptr;
  const int cols8 = (int)(cols / 8);
  const dim3 sgrid((unsigned)((cols + 63) / 64), dbeta ? 2u : 1u);
  if (bwd_one_pass(rows)) {
#define LN_SLAB(NT, J)                                                                                          \
  hipLaunchKernelGGL((ln_bwd_slab_kernel<NT, J>), dim3((unsigned)slabs), dim3(NT), 0, st, x, gamma, mean, rstd, dy, \
                     dres, dx, rows, cols8, (int)cols, part_g, part_b)
    const int snt = bwd_slab_nt(cols);
    const int64_t need = (cols8 + snt - 1) / snt;
    if (snt == 512) {
      if (need == 2) LN_SLAB(512, 2);
      else if (need == 3) LN_SLAB(512, 3);
      else if (need == 4) LN_SLAB(512, 4);
      else return hipErrorInvalidValue;
    } else {
      if (need == 1) LN_SLAB(LN_THREADS, 1);
      else if (need == 2) LN_SLAB(LN_THREADS, 2);
      else return hipErrorInvalidValue;
    }
#undef LN_SLAB
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(slab_sum_kernel, sgrid, blk, 0, st, part_g, dgamma, part_b, dbeta, slabs, cols);
    return hipGetLastError();
  }
  const int64_t strips = (cols + LN_DG_STRIP - 1) / LN_DG_STRIP;
  const int ntiles = (int)(strips * slabs);
  const int nt = ln_nt(rows);
  if (dx != dy) {
    // dx leaves dy intact: the column partials and the dx rows in one launch,
    // then the slab sums
    const int ndg = (ntiles + nt / LN_THREADS - 1) / (nt / LN_THREADS);
    const dim3 grid((unsigned)(ndg + rows)), fb(nt);
#define LN_FEW(NT, J)                                                                                               \
  hipLaunchKernelGGL((ln_bwd_few_kernel<NT, J>), grid, fb, 0, st, x, gamma, mean, rstd, dy, dres, dx, cols8, rows, \
                     cols, rpb, ntiles, ndg, part_g, part_b)
    const int j = ln_j(cols, nt);
    if (nt == 1024) {
      if (j == 1) LN_FEW(1024, 1);
      else if (j == 2) LN_FEW(1024, 2);
      else return hipErrorInvalidValue;
    } else {
      switch (j) {
        case 1: LN_FEW(LN_THREADS, 1); break;
        case 2: LN_FEW(LN_THREADS, 2); break;
        case 3: LN_FEW(LN_THREADS, 3); break;
        case 4: LN_FEW(LN_THREADS, 4); break;
        case 6: LN_FEW(LN_THREADS, 6); break;
        case 8: LN_FEW(LN_THREADS, 8); break;
        default: return hipErrorInvalidValue;
      }
    }
#undef LN_FEW
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(slab_sum_kernel, sgrid, blk, 0, st, part_g, dgamma, part_b, dbeta, slabs, cols);
    return hipGetLastError();
  }
  // dx overwrites dy: the column sums first, as they read dy
  hipLaunchKernelGGL(ln_bwd_dgb_kernel, dim3((unsigned)ntiles), blk, 0, st, x, mean, rstd, dy, rows, cols, rpb,
                     part_g, part_b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(slab_sum_kernel, sgrid, blk, 0, st, part_g, dgamma, part_b, dbeta, slabs, cols);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
#define LN_BWD(NT, J)                                                                                            \
  hipLaunchKernelGGL((ln_bwd_dx_kernel<NT, J>), dim3((unsigned)rows), dim3(NT), 0, st, x, gamma, mean, rstd, dy, \
                     dres, dx, cols8, (int)cols)
  const int j = ln_j(cols, nt);
  if (nt == 1024) {
    if (j == 1) LN_BWD(1024, 1);
    else if (j == 2) LN_BWD(1024, 2);
    else return hipErrorInvalidValue;
  } else {
    switch (j) {
      case 1: LN_BWD(LN_THREADS, 1); break;
      case 2: LN_BWD(LN_THREADS, 2); break;
      case 3: LN_BWD(LN_THREADS, 3); break;
      case 4: LN_BWD(LN_THREADS, 4); break;
      case 6: LN_BWD(LN_THREADS, 6); break;
      case 8: LN_BWD(LN_THREADS, 8); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef LN_BWD
  return hipGetLastError();
}

hipError_t sum_f32_launch(const GradPtrs& g, int t, int64_t n, float* out, hipStream_t st) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  int64_t blocks = (n4 + LN_THREADS - 1) / LN_THREADS;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(sum_f32_kernel, dim3((unsigned)blocks), dim3(LN_THREADS), 0, st, g, t, n4, out);
  return hipGetLastError();
}

}  // namespace tpmlp
