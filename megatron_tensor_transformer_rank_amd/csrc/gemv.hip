// Decode path (one token): split-K GEMV for gfx950, HBM bound.
//
// With one token the up-projection is x @ [Wg_i, W1_i] and the
// down-projection A_i @ W2_i: each weight byte is used exactly once, so the
// kernels are sized to stream the shards from HBM at full rate ("02 -- Tensor
// Parallelism": decode is memory-bandwidth bound work that TP splits across
// HBMs).  No MFMA: every lane owns 8 adjacent output columns, reads 16 bytes
// of a weight row per load (a wave covers 1 KiB of a row, fully coalesced),
// and accumulates in float32 registers.
//
// Grid = strips (512 columns) x matrices x k-splits.  A block's 4 waves take
// interleaved rows of its k range; their sums meet in LDS, the block writes
// one float32 partial row to the workspace, and the last block of a strip to
// finish (device-scope counter, fenced) adds the k-split partials in fixed
// order, applies the epilogue and resets the counter for the next call.  The
// result is deterministic; nothing spins.
#include "common.h"
#include "gemv.h"

namespace tpmlp {

constexpr int GV_THREADS = 256;
constexpr int GV_STRIP = 512;  // columns per block (64 lanes x 8)
constexpr int GV_UNROLL = 8;   // rows in flight per wave per iteration

template <int NMAT, int EPI, int ACT>
__global__ void __launch_bounds__(GV_THREADS)
gemv_splitk(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
            int K, int ncols, int KS, int KR, float* __restrict__ part, unsigned* __restrict__ counters,
            uint16_t* __restrict__ out, uint16_t* __restrict__ st0, uint16_t* __restrict__ st1) {
  __shared__ float xs[GV_MAX_KR];
  __shared__ float red[4][GV_STRIP];
  __shared__ int is_last;

  const int S = (ncols + GV_STRIP - 1) / GV_STRIP;
  const int b = blockIdx.x;
  const int s = b % S;
  const int rest = b / S;
  const int mat = rest % NMAT;
  const int ks = rest / NMAT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  const int kb = ks * KR;
  const int ke = min(K, kb + KR);
  for (int i = tid; i < ke - kb; i += GV_THREADS) xs[i] = bf16_to_f32(x[kb + i]);
  __syncthreads();

  const uint16_t* Wm = (NMAT == 2 && mat == 1) ? W1 : W0;
  const int col = s * GV_STRIP + lane * 8;
  const bool cok = col < ncols;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (cok) {
    const uint16_t* base = Wm + col;
    for (int k = kb + w; k < ke; k += 4 * GV_UNROLL) {
      uint4 v[GV_UNROLL];
#pragma unroll
      for (int u = 0; u < GV_UNROLL; ++u) {
        const int kk = k + 4 * u;
        v[u] = kk < ke ? *reinterpret_cast<const uint4*>(base + (int64_t)kk * ncols) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < GV_UNROLL; ++u) {
        const int kk = k + 4 * u;
        const float xv = kk < ke ? xs[kk - kb] : 0.f;
        acc[0] += xv * bf16lo(v[u].x);
        acc[1] += xv * bf16hi(v[u].x);
        acc[2] += xv * bf16lo(v[u].y);
        acc[3] += xv * bf16hi(v[u].y);
        acc[4] += xv * bf16lo(v[u].z);
        acc[5] += xv * bf16hi(v[u].z);
        acc[6] += xv * bf16lo(v[u].w);
        acc[7] += xv * bf16hi(v[u].w);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = acc[e];
  __syncthreads();

  // block partial: 2 columns per thread, fixed wave order
  float* prow = part + ((int64_t)ks * NMAT + mat) * ncols;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid * 2 + h;
    const int gc = s * GV_STRIP + c;
    if (gc < ncols) prow[gc] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
  }
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const unsigned done = atomicAdd(&counters[s], 1u);
    is_last = done == (unsigned)(KS * NMAT - 1);
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();

#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int c = tid * 2 + h;
    const int gc = s * GV_STRIP + c;
    if (gc >= ncols) continue;
    float sum[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      float a = 0.f;
      for (int q = 0; q < KS; ++q) a += __builtin_nontemporal_load(part + ((int64_t)q * NMAT + m) * ncols + gc);
      sum[m] = a;
    }
    if constexpr (EPI == GV_EPI_STORE) {
      out[gc] = (uint16_t)f32_to_bf16_rne(sum[0]);
    } else if constexpr (EPI == GV_EPI_ACT) {
      out[gc] = (uint16_t)f32_to_bf16_rne(act_f<ACT>(sum[0]));
      if (st0) st0[gc] = (uint16_t)f32_to_bf16_rne(sum[0]);
    } else {  // SwiGLU: matrix 0 = gate, matrix 1 = up
      out[gc] = (uint16_t)f32_to_bf16_rne(swiglu_f(sum[0], sum[NMAT - 1]));
      if (st0) st0[gc] = (uint16_t)f32_to_bf16_rne(sum[0]);
      if (st1) st1[gc] = (uint16_t)f32_to_bf16_rne(sum[NMAT - 1]);
    }
  }
  if (tid == 0) counters[s] = 0u;
}

GemvPlan gemv_plan(int K, int ncols, int nmat, int num_cu) {
  GemvPlan p;
  p.strips = (ncols + GV_STRIP - 1) / GV_STRIP;
  // aim for ~4 blocks per CU, at least 64 rows per block, KR <= GV_MAX_KR
  const int target = 4 * num_cu;
  int ks = (target + p.strips * nmat - 1) / (p.strips * nmat);
  ks = max(1, min(ks, (K + 63) / 64));
  int kr = (K + ks - 1) / ks;
  kr = ((kr + 3) / 4) * 4;
  if (kr > GV_MAX_KR) kr = GV_MAX_KR;
  ks = (K + kr - 1) / kr;
  p.ks = ks;
  p.kr = kr;
  p.part_floats = (size_t)ks * nmat * ncols;
  return p;
}

hipError_t gemv_launch(int epi, int act, const uint16_t* x, const uint16_t* W0, const uint16_t* W1, int K,
                       int ncols, const GemvPlan& p, float* part, unsigned* counters, uint16_t* out,
                       uint16_t* st0, uint16_t* st1, hipStream_t st) {
  const int nmat = epi == GV_EPI_SWIGLU ? 2 : 1;
  const dim3 grid((unsigned)(p.strips * nmat * p.ks)), block(GV_THREADS);
  if (epi == GV_EPI_SWIGLU)
    hipLaunchKernelGGL((gemv_splitk<2, GV_EPI_SWIGLU, ACT_SWIGLU>), grid, block, 0, st, x, W0, W1, K, ncols, p.ks,
                       p.kr, part, counters, out, st0, st1);
  else if (epi == GV_EPI_ACT && act == ACT_RELU)
    hipLaunchKernelGGL((gemv_splitk<1, GV_EPI_ACT, ACT_RELU>), grid, block, 0, st, x, W0, W1, K, ncols, p.ks, p.kr,
                       part, counters, out, st0, st1);
  else if (epi == GV_EPI_ACT)
    hipLaunchKernelGGL((gemv_splitk<1, GV_EPI_ACT, ACT_GELU>), grid, block, 0, st, x, W0, W1, K, ncols, p.ks, p.kr,
                       part, counters, out, st0, st1);
  else
    hipLaunchKernelGGL((gemv_splitk<1, GV_EPI_STORE, 0>), grid, block, 0, st, x, W0, W1, K, ncols, p.ks, p.kr, part,
                       counters, out, st0, st1);
  return hipGetLastError();
}

}  // namespace tpmlp
