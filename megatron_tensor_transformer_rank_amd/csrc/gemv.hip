// Decode path (one token): split-K GEMVs for gfx950, HBM bound.
//
// With one token the up-projection is x @ [Wg_i, W1_i] and the
// down-projection A_i @ W2_i: each weight byte is used exactly once, so the
// kernels are built to stream the shards from HBM at full rate ("02 -- Tensor
// Parallelism": decode is memory-bandwidth bound work that TP splits across
// HBMs).  No MFMA: every lane owns 8 adjacent output columns, reads 16 bytes
// of a weight row per load (a wave covers 1 KiB of a row, fully coalesced),
// with non-temporal loads (streamed data is not kept in the caches), and
// accumulates in float32 registers.
//
// Two launches.  No block waits for another; the down-projection's k-split
// partials are summed by the last block of each column strip to finish (an
// agent-scope fence per block, which writes back the XCD's whole L2, costs
// more than the whole stream, so the partials go through device-scope
// stores and loads instead, see gemv_partial):
//   1. up:    blocks = 512-column strips x matrices x k-splits; a block's 16
//             waves take interleaved rows of its k range, each lane keeping 8
//             weight loads in flight in a rolling pipeline; the waves meet in
//             LDS and write one float32 partial row per (k-split, matrix).
//   2. down:  same streaming over W2_i, about one block per CU (fewer, longer
//             blocks stream this shape faster than 1-2 per CU); its prologue
//             adds the up-projection's k-split partials for the block's rows
//             in fixed order, applies the activation and rounds A to bf16
//             (the value the MFMA path would read back), while the block's
//             first weight loads are in flight.  Blocks of the first column
//             strip also write A_i and the stash.  The last block of each
//             strip adds the strip's k-split partials in fixed order and
//             rounds Y_i to bf16.
// The result is deterministic.
#include "common.h"
#include "gemv.h"

namespace tpmlp {

constexpr int GV_WAVES = 16;
constexpr int GV_THREADS = 64 * GV_WAVES;
constexpr int GV_STRIP = 512;  // columns per block (64 lanes x 8)
constexpr int GV_UNROLL = 8;   // weight loads in flight per lane
constexpr int GV_FINAL_COLS = 128;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_stream(const uint16_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// PRO = 0: x is the bf16 input vector.  PRO = 1: x[k] = act(sum of the
// up-projection partials pg[q][*][k]) rounded to bf16 (ACT selects ReLU /
// GeLU over one matrix or SwiGLU over gate and up).
//
// Wave w of the block takes rows kb + w, kb + w + GV_WAVES, ...; its weight
// loads form a rolling pipeline: slot u holds row j = step * GV_UNROLL + u,
// and is refilled with row j + GV_UNROLL as soon as it has been consumed, so
// GV_UNROLL loads stay in flight per lane through the whole k range.
//
// FIN = 1 (the down-projection): the block's partial row is written with
// device-scope stores (they reach the memory side that every XCD sees, past
// the XCD's own L2), the block waits for them to complete and then bumps its
// strip's counter; the block that finds every other k-split of its strip
// counted is the last one, and adds the strip's partials (read with
// device-scope loads) in k-split order into Y, then zeroes the counter.  The
// counters are zeroed beforehand by the up-projection kernel of the same
// call (zero_cnt), so the workspace needs no initial contents.
template <int NMAT, int PRO, int ACT, int FIN>
__global__ void __launch_bounds__(GV_THREADS)
gemv_partial(const uint16_t* __restrict__ x, const uint16_t* __restrict__ W0, const uint16_t* __restrict__ W1,
             int K, int ncols, int KR, float* __restrict__ part, const float* __restrict__ pg, int ks_up,
             uint16_t* __restrict__ a_out, uint16_t* __restrict__ st0, uint16_t* __restrict__ st1,
             int* __restrict__ cnt, int ncnt, uint16_t* __restrict__ y) {
  __shared__ float xs[GV_MAX_KR];
  __shared__ float red[GV_WAVES][GV_STRIP];
  __shared__ int last;

  const int S = (ncols + GV_STRIP - 1) / GV_STRIP;
  const int b = blockIdx.x;
  const int s = b % S;
  const int rest = b / S;
  const int mat = rest % NMAT;
  const int ks = rest / NMAT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int kb = ks * KR;
  const int ke = min(K, kb + KR);

  const uint16_t* Wm = (NMAT == 2 && mat == 1) ? W1 : W0;
  if (PRO == 0 && cnt != nullptr && b == 0)  // the next kernel's strip counters start at zero
    for (int i = tid; i < ncnt; i += GV_THREADS) __hip_atomic_store(cnt + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int col = s * GV_STRIP + lane * 8;
  const bool cok = col < ncols;
  const uint16_t* base = Wm + col + (int64_t)(kb + w) * ncols;
  const int64_t rstride = (int64_t)GV_WAVES * ncols;
  const int nrows = cok && ke - kb > w ? (ke - kb - w + GV_WAVES - 1) / GV_WAVES : 0;  // rows of this lane

  // first loads before x is staged: they do not depend on it
  u32x4 v[GV_UNROLL];
#pragma unroll
  for (int u = 0; u < GV_UNROLL; ++u) v[u] = u < nrows ? ld_stream(base + u * rstride) : u32x4{0u, 0u, 0u, 0u};

  if constexpr (PRO == 0) {
    for (int i = tid; i < ke - kb; i += GV_THREADS) xs[i] = bf16_to_f32(x[kb + i]);
  } else {
    constexpr int NU = ACT == ACT_SWIGLU ? 2 : 1;
    for (int i = tid; i < ke - kb; i += GV_THREADS) {
      const int kk = kb + i;
      float sum[NU];
#pragma unroll
      for (int m = 0; m < NU; ++m) sum[m] = 0.f;
      // all partial loads of a batch in flight at once, added in k-split order
      constexpr int QB = 16;
      for (int q0 = 0; q0 < ks_up; q0 += QB) {
        float pv[QB][NU];
#pragma unroll
        for (int u = 0; u < QB; ++u)
#pragma unroll
          for (int m = 0; m < NU; ++m)
            pv[u][m] = q0 + u < ks_up ? pg[((int64_t)(q0 + u) * NU + m) * K + kk] : 0.f;
#pragma unroll
        for (int u = 0; u < QB; ++u)
#pragma unroll
          for (int m = 0; m < NU; ++m) sum[m] += pv[u][m];
      }
      float a;
      if constexpr (ACT == ACT_SWIGLU) a = swiglu_f(sum[0], sum[1]);
      else a = act_f<ACT>(sum[0]);
      const uint32_t ab = f32_to_bf16_rne(a);
      xs[i] = __uint_as_float(ab << 16);
      if (s == 0) {
        a_out[kk] = (uint16_t)ab;
        if (st0) st0[kk] = (uint16_t)f32_to_bf16_rne(sum[0]);
        if (ACT == ACT_SWIGLU && st1) st1[kk] = (uint16_t)f32_to_bf16_rne(sum[NU - 1]);
      }
    }
  }
  __syncthreads();

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int nsteps = (nrows + GV_UNROLL - 1) / GV_UNROLL;
  for (int step = 0; step < nsteps; ++step) {
#pragma unroll
    for (int u = 0; u < GV_UNROLL; ++u) {
      const int j = step * GV_UNROLL + u;
      const float xv = j < nrows ? xs[w + GV_WAVES * j] : 0.f;
      const u32x4 c = v[u];
      acc[0] += xv * bf16lo(c.x);
      acc[1] += xv * bf16hi(c.x);
      acc[2] += xv * bf16lo(c.y);
      acc[3] += xv * bf16hi(c.y);
      acc[4] += xv * bf16lo(c.z);
      acc[5] += xv * bf16hi(c.z);
      acc[6] += xv * bf16lo(c.w);
      acc[7] += xv * bf16hi(c.w);
      const int jn = j + GV_UNROLL;
      v[u] = jn < nrows ? ld_stream(base + jn * rstride) : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[w][lane * 8 + e] = acc[e];
  __syncthreads();

  // block partial row: waves added in fixed order
  for (int c = tid; c < GV_STRIP; c += GV_THREADS) {
    const int gc = s * GV_STRIP + c;
    if (gc < ncols) {
      float t = red[0][c];
#pragma unroll
      for (int q = 1; q < GV_WAVES; ++q) t += red[q][c];
      float* dst = part + ((int64_t)ks * NMAT + mat) * ncols + gc;
      if constexpr (FIN) __hip_atomic_store(dst, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *dst = t;
    }
  }
  if constexpr (FIN) {
    const int nks = gridDim.x / S;  // k-splits of this strip (NMAT = 1)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's partial stores have completed
    __syncthreads();
    if (tid == 0) last = __hip_atomic_fetch_add(cnt + s, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nks - 1;
    __syncthreads();
    if (last) {
      for (int c = tid; c < GV_STRIP; c += GV_THREADS) {
        const int gc = s * GV_STRIP + c;
        if (gc >= ncols) continue;
        float t = 0.f;
        constexpr int QB = 16;
        for (int q0 = 0; q0 < nks; q0 += QB) {
          float pv[QB];
#pragma unroll
          for (int u = 0; u < QB; ++u)
            pv[u] = q0 + u < nks ? __hip_atomic_load(part + (int64_t)(q0 + u) * ncols + gc, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT)
                                 : 0.f;
#pragma unroll
          for (int u = 0; u < QB; ++u) t += pv[u];
        }
        y[gc] = (uint16_t)f32_to_bf16_rne(t);
      }
      if (tid == 0) __hip_atomic_store(cnt + s, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// out[c] = bf16(sum_q part[q][c]).  A block owns GV_FINAL_COLS columns; its
// 8 thread groups each add every 8th partial in increasing q, then group
// sums are added in group order: a fixed order, so the result is
// deterministic.
__global__ void __launch_bounds__(256)
gemv_final(const float* __restrict__ part, int ks, int ncols, uint16_t* __restrict__ out) {
  __shared__ float4 red[8][GV_FINAL_COLS / 4];
  const int c4 = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int c = blockIdx.x * GV_FINAL_COLS + c4 * 4;
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < ncols) {
    constexpr int TU = 4;
    for (int q0 = grp; q0 < ks; q0 += 8 * TU) {
      float4 t[TU];
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        const int q = q0 + 8 * u;
        t[u] = q < ks ? *reinterpret_cast<const float4*>(part + (int64_t)q * ncols + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < TU; ++u) {
        a.x += t[u].x; a.y += t[u].y; a.z += t[u].z; a.w += t[u].w;
      }
    }
  }
  red[grp][c4] = a;
  __syncthreads();
  if (grp == 0 && c < ncols) {
    float4 r = red[0][c4];
#pragma unroll
    for (int q = 1; q < 8; ++q) {
      const float4 o = red[q][c4];
      r.x += o.x; r.y += o.y; r.z += o.z; r.w += o.w;
    }
    *reinterpret_cast<uint2*>(out + c) = make_uint2(pack_bf16x2(r.x, r.y), pack_bf16x2(r.z, r.w));
  }
}

GemvPlan gemv_plan(int K, int ncols, int nmat, int target_blocks) {
  GemvPlan p;
  p.strips = (ncols + GV_STRIP - 1) / GV_STRIP;
  int ks = (target_blocks + p.strips * nmat - 1) / (p.strips * nmat);
  ks = max(1, min(ks, (K + GV_WAVES - 1) / GV_WAVES));
  int kr = (K + ks - 1) / ks;
  kr = ((kr + GV_WAVES - 1) / GV_WAVES) * GV_WAVES;  // whole rows for every wave
  if (kr > GV_MAX_KR) kr = GV_MAX_KR;
  p.ks = (K + kr - 1) / kr;
  p.kr = kr;
  p.part_floats = (size_t)p.ks * nmat * ncols;
  return p;
}

hipError_t decode_launch(int act, const uint16_t* x, const uint16_t* Wa, const uint16_t* Wb, const uint16_t* W2,
                         int h, int Fi, const GemvPlan& up, const GemvPlan& down, float* part_up, float* part_down,
                         int* cnt, uint16_t* A, uint16_t* st0, uint16_t* st1, uint16_t* Y, hipStream_t st) {
  const dim3 blk(GV_THREADS);
  if (act == ACT_SWIGLU) {
    hipLaunchKernelGGL((gemv_partial<2, 0, 0, 0>), dim3(up.strips * 2 * up.ks), blk, 0, st, x, Wa, Wb, h, Fi, up.kr,
                       part_up, nullptr, 0, nullptr, nullptr, nullptr, cnt, down.strips, nullptr);
  } else {
    hipLaunchKernelGGL((gemv_partial<1, 0, 0, 0>), dim3(up.strips * up.ks), blk, 0, st, x, Wa, Wa, h, Fi, up.kr,
                       part_up, nullptr, 0, nullptr, nullptr, nullptr, cnt, down.strips, nullptr);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 gd(down.strips * down.ks);
  if (act == ACT_SWIGLU)
    hipLaunchKernelGGL((gemv_partial<1, 1, ACT_SWIGLU, 1>), gd, blk, 0, st, nullptr, W2, W2, Fi, h, down.kr,
                       part_down, part_up, up.ks, A, st0, st1, cnt, down.strips, Y);
  else if (act == ACT_RELU)
    hipLaunchKernelGGL((gemv_partial<1, 1, ACT_RELU, 1>), gd, blk, 0, st, nullptr, W2, W2, Fi, h, down.kr, part_down,
                       part_up, up.ks, A, st0, nullptr, cnt, down.strips, Y);
  else
    hipLaunchKernelGGL((gemv_partial<1, 1, ACT_GELU, 1>), gd, blk, 0, st, nullptr, W2, W2, Fi, h, down.kr, part_down,
                       part_up, up.ks, A, st0, nullptr, cnt, down.strips, Y);
  return hipGetLastError();
}

hipError_t ksum_launch(const float* part, int ks, int64_t n, uint16_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gemv_final, dim3((unsigned)((n + GV_FINAL_COLS - 1) / GV_FINAL_COLS)), dim3(256), 0, st, part, ks,
                     (int)n, out);
  return hipGetLastError();
}

}  // namespace tpmlp
