// Small-batch path (up to 128 tokens): split-K MFMA GEMMs for gfx950 that
// stream each weight once -- the forward for 2 <= N <= 128 and the
// backward's input gradients for 1 <= N <= 128.
//
// With a handful of tokens every weight byte is still used by only N
// multiply-adds, so the forward is bound by reading the shards from HBM, as
// in one-token decode ("02 -- Tensor Parallelism": decode is memory-bandwidth
// bound work that TP splits across HBMs; batch sizes below ~32 stay in that
// regime).  The wide-tile GEMM would cover the 70B-class shard's up
// projection with only 56 column tiles; here every 256-column strip of a
// weight is also split along k so that about one block runs per CU, each
// streaming its [k-range x 256] slab through LDS.  Up to 128 tokens this
// stays 2.2-2.6x faster than the wide tiles at the 7B-, 70B- and GPT-3-class
// shards, whose 128-row tiles leave most CUs idle there.
//
//   1. skinny_partial (up):   X [N, h] @ W (gate and up side by side for
//                             SwiGLU) -> float32 partials [ks][mat][N][F_i]
//   2. skinny_act:            A = act(sum of the partials in k-split order),
//                             rounded to bf16, plus the pre-activation stashes
//   3. skinny_partial (down): A [N, F_i] @ W2 -> partials [ks][N][h]
//   4. k-split sum:           Y = bf16(sum of the partials), the one-token
//                             path's final reduction
//
// The backward's input gradients read their weights k-contiguous as stored
// (NT: W2 [F_i, h] and W1, Wg [h, F_i] are [output column][k]), with the
// partials in the weight gradient's storage (the caller writes it later):
//   dU: skinny_partial<.., 1, NT> (dY @ W2^T), then skinny_act_bwd (the sum,
//       then dU = dA * act'(U), SwiGLU's [dG | dP] from G and U);
//   dX: skinny_partial<.., g, NT> (dU @ W1^T; SwiGLU's dG @ Wg^T and
//       dP @ W1^T as matrices 0 and 1), then the k-split sum over both.
//
// skinny_partial: 4 waves (8 at 128 rows: two groups of 4, each owning 64 of
// the rows); the block's tile is MB token rows (N padded to 16, 32, 64 or
// 128; or, when the weights are too small to give every CU a block, tiles of
// 32 or 64 of the rows, the grid's second dimension) x 256 columns, each
// wave owning 64 columns.  Four LDS stages (three at 128 rows), each [64 k][256] of the
// weight (n-contiguous, read with the LDS transpose read; with NT [256][64 k],
// k-contiguous like the activations and read with ds_read_b128) and
// [MB][64 k] of the activations; the DMA of tile t+3 (t+2) is issued as tile
// t's fragments are read, so about 100 KiB per CU stay in flight.  One barrier per 64-deep
// k-tile.  The MFMA work per byte is small (2*MB flops per weight element).
#include "common.h"
#include "gemv.h"
#include "skinny.h"
#include "tiles.h"

namespace tpmlp {

constexpr int SK_COLS = 256;  // columns per block
constexpr int SK_BK = 64;
constexpr int SK_QB = 8;  // k-split partials loaded together by the activation kernels

// Waves per block: 4, or 8 for 128 token rows (two groups of four, each
// owning 64 of the rows), so that each SIMD runs two waves and one's LDS
// reads and waits overlap the other's MFMAs.
template <int MB>
constexpr int sk_waves() { return MB == 128 ? 8 : 4; }

template <int MB, int NMAT, bool NT>
__global__ void __launch_bounds__(64 * sk_waves<MB>())
skinny_partial(const uint16_t* __restrict__ X, int N, int64_t ldx, uint32_t x_bytes, int64_t x1_off,
               const uint16_t* W0, const uint16_t* W1, uint32_t w_bytes, int K, int ncols, int strips,
               int kt_per_split, float* __restrict__ part) {
  constexpr int GROUPS = sk_waves<MB>() / 4;  // wave groups, each owning MB / GROUPS rows
  constexpr int TM = MB / 16 / GROUPS;        // 16-row blocks per wave
  constexpr int TN = 4;                       // 16-column blocks per wave
  constexpr int W_BYTES = SK_COLS * 128;     // [64 k][256 cols]
  constexpr int NIX = MB / 32 > 0 ? MB / 32 : 1;  // activation DMA instructions per wave
  constexpr int X_BYTES = NIX * 4 * 1024;   // [MB rows][64 k], rounded up to whole instructions
  constexpr int STAGE = W_BYTES + X_BYTES;
  // four LDS stages (three tiles in flight); three (two in flight) for 128
  // token rows, whose activation tile doubles the stage
  constexpr int SK_STAGES = MB == 128 ? 3 : 4;
  constexpr int NIW = SK_COLS / 32;          // weight DMA instructions per wave of a group
  constexpr int NI = (NIW + NIX) / GROUPS;   // DMA instructions a wave issues per tile
  __shared__ __attribute__((aligned(1024))) uint8_t smem[SK_STAGES * STAGE];

  const int lane = threadIdx.x & 63;
  // wave w of group grp: columns 64 w .. of the tile, rows grp * MB / GROUPS ..;
  // the group's DMA share is every GROUPS-th block of the four-wave pattern
  const int wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = wg & 3, grp = wg >> 2;
  const int b = blockIdx.x;
  const int s = b % strips, rest = b / strips;
  const int mat = rest % NMAT, q = rest / NMAT;
  const int col0 = s * SK_COLS;
  const int nkt = (K + SK_BK - 1) / SK_BK;
  const int t0 = q * kt_per_split;
  const int nt = min(nkt, t0 + kt_per_split) - t0;
  const uint16_t* Wm = (NMAT == 2 && mat == 1) ? W1 : W0;

  // weight tile DMA: [64 k][256 cols] of Wm from k-row k0 (Wm is [K][ncols]),
  // or with NT the 256 rows col0.. of Wm [ncols][K] from column k0, stored
  // k-contiguous like the activations
  DmaMN<SK_COLS> dw;
  DmaK<SK_COLS> dwk;
  if constexpr (NT)
    dwk.init(col0, ncols, K, lane, w);
  else
    dw.init(col0, ncols, ncols, lane, w);
  const uint32_t wk_step = NT ? 2u : (uint32_t)ncols * 2u;  // bytes per k of the weight tile's origin
  // activation tile DMA: instruction i = w + 4j covers rows 8i .. 8i+7, eight
  // 16-byte chunks per row, chunk c of row r at slot c ^ (r & 7); rows past N
  // (and the padding instructions when MB = 16) read zeros.  Matrix 1 of a
  // pair whose activations sit side by side in one buffer reads from column
  // x1_off.
  const int kc = ((lane & 7) ^ ((lane >> 3) & 7)) * 8;
  const int row0 = blockIdx.y * MB;  // the block's row tile
  const uint32_t xcol = (uint32_t)((mat == 1 ? x1_off : 0) * 2);
  uint32_t xoff[NIX];
#pragma unroll
  for (int j = 0; j < NIX; ++j) {
    const int row = (w + 4 * j) * 8 + (lane >> 3);
    xoff[j] = (row0 + row < N && row < MB) ? (uint32_t)((int64_t)(row0 + row) * ldx * 2) + xcol + (uint32_t)kc * 2u
                                           : OOB;
  }
  auto shifted = [](const uint16_t* p, uint32_t bytes, uint32_t skip) __attribute__((always_inline)) {
    const uint64_t a = reinterpret_cast<uint64_t>(p) + skip;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(skip < bytes ? bytes - skip : 0u);
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
  };
  // DMA of the split's i-th tile into stage slot; tiles past the split read
  // zeros (keeps the per-wave count of loads in flight uniform)
  auto issue_tile = [&](int i, uint8_t* st) __attribute__((always_inline)) {
    const bool live = i < nt;
    const int k0 = (t0 + i) * SK_BK;
    const int kvalid = live ? K - k0 : 0;
    const rsrc_t rw = shifted(Wm, live ? w_bytes : 0u, (uint32_t)k0 * wk_step);
    static_for<NIW>([&](auto J) __attribute__((always_inline)) {
      constexpr int jj = decltype(J)::value;
      if (GROUPS == 1 || jj / (NIW / GROUPS) == grp) {
        if constexpr (NT)
          dwk.template issue<jj>(rw, st, kvalid, w);
        else
          dw.template issue<jj>(rw, st, w);
      }
    });
    const rsrc_t rx = shifted(X, live ? x_bytes : 0u, (uint32_t)k0 * 2u);
#pragma unroll
    for (int j = 0; j < NIX; ++j)
      if (GROUPS == 1 || j / (NIX / GROUPS) == grp)
        dma16(rx, st + W_BYTES + (w + 4 * j) * 1024, kc < kvalid ? xoff[j] : OOB);
  };

  // fragment addressing within a stage
  const uint32_t a_row0 = W_BYTES + (uint32_t)grp * TM * 2048;  // the group's first row block
  const uint32_t a_off0 = a_row0 + kfrag_off(0, 0, lane), a_off1 = a_row0 + kfrag_off(0, 1, lane);
  uint32_t b_col[TN];
  if constexpr (NT) {
    b_col[0] = kfrag_off(w * 64, 0, lane);
    b_col[1] = kfrag_off(w * 64, 1, lane);
  } else {
    const uint32_t kb = mn_kbase<SK_COLS>(lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) b_col[j] = kb + mn_coloff<SK_COLS>(w * 64, j, lane);
  }

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t base = lds_addr(smem);
#pragma unroll
  for (int p = 0; p < SK_STAGES - 1; ++p) issue_tile(p, smem + p * STAGE);

  for (int i = 0; i < nt; ++i) {
    const int sl = i % SK_STAGES;
    // this wave's loads of tile i have landed; after the barrier everyone's
    // have, and everyone has finished reading tile i-1's slot
    wait_vmcnt<(SK_STAGES - 2) * NI>();
    barrier();
    const int sn = (i + SK_STAGES - 1) % SK_STAGES;
    issue_tile(i + SK_STAGES - 1, smem + sn * STAGE);
    const uint32_t sa = base + sl * STAGE;
    bf16x8 af[2][TM], bf[2][TN];
    static_for<TM>([&](auto I) __attribute__((always_inline)) {
      constexpr int ii = decltype(I)::value;
      af[0][ii] = ld_b128<ii * 2048>(sa + a_off0);
      af[1][ii] = ld_b128<ii * 2048>(sa + a_off1);
    });
    constexpr int RS = SK_COLS * 2;
    static_for<TN>([&](auto J) __attribute__((always_inline)) {
      constexpr int jj = decltype(J)::value;
      if constexpr (NT) {
        bf[0][jj] = ld_b128<jj * 2048>(sa + b_col[0]);
        bf[1][jj] = ld_b128<jj * 2048>(sa + b_col[1]);
      } else {
        bf[0][jj] = ld_tr2<0, 4 * RS>(sa + b_col[jj]);
        bf[1][jj] = ld_tr2<32 * RS, 36 * RS>(sa + b_col[jj]);
      }
    });
    // the fragments are consumed only after this wait: the reads and MFMAs
    // are volatile asm, so they keep this order
    wait_lgkm0();
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int ii = 0; ii < TM; ++ii)
#pragma unroll
        for (int jj = 0; jj < TN; ++jj)
          asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc[ii][jj]) : "v"(bf[st][jj]), "v"(af[st][ii]));
  }
  asm volatile("s_nop 15\n\ts_nop 7" ::: "memory");  // last MFMA results written before they are read
  wait_vmcnt<0>();  // no DMA may land after the block has left

  // lane holds rows n = row0 + grp * 16 TM + 16i + l16, columns col0 + 64w + 16j + 4lq .. +3
  const int l16 = lane & 15, lq = lane >> 4;
  float* dst = part + (int64_t)(q * NMAT + mat) * N * ncols;
#pragma unroll
  for (int ii = 0; ii < TM; ++ii) {
    const int n = row0 + (grp * TM + ii) * 16 + l16;
    if (n >= N) continue;
#pragma unroll
    for (int jj = 0; jj < TN; ++jj) {
      const int c = col0 + w * 64 + jj * 16 + 4 * lq;
      if (c < ncols)
        *reinterpret_cast<float4*>(dst + (int64_t)n * ncols + c) =
            make_float4(acc[ii][jj][0], acc[ii][jj][1], acc[ii][jj][2], acc[ii][jj][3]);
    }
  }
}

// A[e] = act(sum_q part[q][0][e] (, sum_q part[q][1][e])) for e < n (the
// flattened [N, F_i]); sums in k-split order.  st0 / st1 as for the decode
// GEMVs (SwiGLU: gate, up; otherwise st0 = the pre-activation).
template <int ACT>
__global__ void __launch_bounds__(256)
skinny_act(const float* __restrict__ part, int ks, int64_t n, uint16_t* __restrict__ A, uint16_t* __restrict__ st0,
           uint16_t* __restrict__ st1) {
  constexpr int NMAT = ACT == ACT_SWIGLU ? 2 : 1;
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < n; e += (int64_t)gridDim.x * 256 * 4) {
    float4 sum[NMAT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m) sum[m] = make_float4(0.f, 0.f, 0.f, 0.f);
    // SK_QB splits' loads in flight at a time, then added in split order
    for (int q0 = 0; q0 < ks; q0 += SK_QB) {
      float4 v[SK_QB][NMAT];
#pragma unroll
      for (int u = 0; u < SK_QB; ++u)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          v[u][m] = q0 + u < ks ? *reinterpret_cast<const float4*>(part + ((int64_t)(q0 + u) * NMAT + m) * n + e)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < SK_QB; ++u)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
          if (q0 + u < ks) {
            sum[m].x += v[u][m].x; sum[m].y += v[u][m].y; sum[m].z += v[u][m].z; sum[m].w += v[u][m].w;
          }
    }
    float a[4];
    const float g[4] = {sum[0].x, sum[0].y, sum[0].z, sum[0].w};
    const float u[4] = {sum[NMAT - 1].x, sum[NMAT - 1].y, sum[NMAT - 1].z, sum[NMAT - 1].w};
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = ACT == ACT_SWIGLU ? swiglu_f(g[r], u[r]) : act_f<ACT>(g[r]);
    *reinterpret_cast<uint2*>(A + e) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
    if (st0) *reinterpret_cast<uint2*>(st0 + e) = make_uint2(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]));
    if (ACT == ACT_SWIGLU && st1)
      *reinterpret_cast<uint2*>(st1 + e) = make_uint2(pack_bf16x2(u[0], u[1]), pack_bf16x2(u[2], u[3]));
  }
}

// Backward through the activation: dA[e] = sum_q part[q][e] (k-split order)
// over the flattened [N, F_i], then dU = dA * act'(U) (bf16 [N, F_i]), or for
// SwiGLU the row [dG | dP] of dU [N, 2 F_i] from the stashes G, U.  The same
// arithmetic as the wide-tile GEMM's epilogue, on a differently ordered dA.
template <int ACT>
__global__ void __launch_bounds__(256)
skinny_act_bwd(const float* __restrict__ part, int ks, int64_t n, int Fi, const uint16_t* __restrict__ U,
               const uint16_t* __restrict__ G, uint16_t* __restrict__ dU) {
  for (int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; e < n; e += (int64_t)gridDim.x * 256 * 4) {
    // the stashes' loads first, then SK_QB splits' loads in flight at a time,
    // added in split order
    const uint2 ub = *reinterpret_cast<const uint2*>(U + e);
    const uint2 gb = ACT == ACT_SWIGLU ? *reinterpret_cast<const uint2*>(G + e) : make_uint2(0u, 0u);
    float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int q0 = 0; q0 < ks; q0 += SK_QB) {
      float4 v[SK_QB];
#pragma unroll
      for (int u = 0; u < SK_QB; ++u)
        v[u] = q0 + u < ks ? *reinterpret_cast<const float4*>(part + (int64_t)(q0 + u) * n + e)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < SK_QB; ++u)
        if (q0 + u < ks) {
          sum.x += v[u].x; sum.y += v[u].y; sum.z += v[u].z; sum.w += v[u].w;
        }
    }
    const float da[4] = {sum.x, sum.y, sum.z, sum.w};
    const float uu[4] = {bf16lo(ub.x), bf16hi(ub.x), bf16lo(ub.y), bf16hi(ub.y)};
    if constexpr (ACT == ACT_SWIGLU) {
      const float gg[4] = {bf16lo(gb.x), bf16hi(gb.x), bf16lo(gb.y), bf16hi(gb.y)};
      float dg[4], dp[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) swiglu_grad_f(da[r], gg[r], uu[r], dg[r], dp[r]);
      // F_i % 8 == 0: the four elements share one row
      const int64_t row = e / Fi, f = e - row * Fi;
      uint16_t* out = dU + row * 2 * Fi + f;
      *reinterpret_cast<uint2*>(out) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
      *reinterpret_cast<uint2*>(out + Fi) = make_uint2(pack_bf16x2(dp[0], dp[1]), pack_bf16x2(dp[2], dp[3]));
    } else {
      float d[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = da[r] * act_grad_f<ACT>(uu[r]);
      *reinterpret_cast<uint2*>(dU + e) = make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
    }
  }
}

SkinnyPlan skinny_plan(int N, int K, int ncols, int nmat, int target_blocks, int max_ks) {
  SkinnyPlan p;
  p.rows = N <= 16 ? 16 : (N <= 32 ? 32 : (N <= 64 ? 64 : 128));
  p.strips = (ncols + SK_COLS - 1) / SK_COLS;
  const int nkt = (K + SK_BK - 1) / SK_BK;
  // no more splits than keep the float32 partials (ks N ncols 4 bytes) within
  // the weight's own bytes (K ncols 2): past that, writing and re-reading them
  // costs more than the extra blocks gain (at 128 tokens and h = 1024 the
  // forward took 29.9 us with 4 and 8 splits against 31.9 with 16 and 32)
  const int traffic_ks = max(1, K / (2 * N));
  int ks = target_blocks / (p.strips * nmat);
  ks = max(1, min(min(min(ks, max_ks), traffic_ks), nkt));
  p.kt = (nkt + ks - 1) / ks;
  p.ks = (nkt + p.kt - 1) / p.kt;  // every split non-empty
  p.part_floats = (size_t)p.ks * nmat * N * ncols;
  // A grid well below the target (small weights: few strips, few splits
  // under the caps) takes the rows in tiles of 32 (else 64), as many tiles as
  // fit the target.  Each row tile reads the whole weight tile again, which
  // at these sizes the caches hold.  Measured on the 128-token training
  // shard (h = 1024, F_i = 2048): step 65.5 -> 50.5 us from a graph (32 of
  // 256 blocks per product before).
  p.rtiles = 1;
  const int blocks = p.strips * nmat * p.ks;
  const int rt_max = target_blocks / blocks;
  if (rt_max >= 2 && N > 32) {
    if ((N + 31) / 32 <= rt_max) {
      p.rows = 32;
      p.rtiles = (N + 31) / 32;
    } else if (N > 64 && (N + 63) / 64 <= rt_max) {
      p.rows = 64;
      p.rtiles = (N + 63) / 64;
    }
  }
  return p;
}

namespace {

// x1_off: the element offset of matrix 1's activations from X (NMAT = 2
// with NT: two k segments whose activations sit side by side in one row)
template <int NMAT, bool NT, int MB>
void partial_one(const SkinnyPlan& p, dim3 grid, int N, const uint16_t* X, int64_t ldx, uint32_t x_bytes,
                 int64_t x1_off, const uint16_t* W0, const uint16_t* W1, uint32_t w_bytes, int K, int ncols,
                 float* part, hipStream_t st) {
  hipLaunchKernelGGL((skinny_partial<MB, NMAT, NT>), grid, dim3(64 * sk_waves<MB>()), 0, st, X, N, ldx, x_bytes,
                     x1_off, W0, W1, w_bytes, K, ncols, p.strips, p.kt, part);
}

template <int NMAT, bool NT>
hipError_t partial_launch(const SkinnyPlan& p, int N, const uint16_t* X, int64_t ldx, int64_t x1_off,
                          const uint16_t* W0, const uint16_t* W1, int K, int ncols, float* part, hipStream_t st) {
  const uint32_t x_bytes = (uint32_t)((int64_t)N * ldx * 2);
  const uint32_t w_bytes = (uint32_t)((int64_t)K * ncols * 2);
  const dim3 grid(p.strips * NMAT * p.ks, p.rtiles);
  if (p.rows == 16)
    partial_one<NMAT, NT, 16>(p, grid, N, X, ldx, x_bytes, x1_off, W0, W1, w_bytes, K, ncols, part, st);
  else if (p.rows == 32)
    partial_one<NMAT, NT, 32>(p, grid, N, X, ldx, x_bytes, x1_off, W0, W1, w_bytes, K, ncols, part, st);
  else if (p.rows == 64)
    partial_one<NMAT, NT, 64>(p, grid, N, X, ldx, x_bytes, x1_off, W0, W1, w_bytes, K, ncols, part, st);
  else
    partial_one<NMAT, NT, 128>(p, grid, N, X, ldx, x_bytes, x1_off, W0, W1, w_bytes, K, ncols, part, st);
  return hipGetLastError();
}

int act_blocks(int64_t n) {
  const int64_t b = (n / 4 + 255) / 256;
  return (int)(b < 1024 ? (b < 1 ? 1 : b) : 1024);
}

}  // namespace

hipError_t skinny_launch(int act, int N, const uint16_t* X, const uint16_t* Wa, const uint16_t* Wb,
                         const uint16_t* W2, int h, int Fi, const SkinnyPlan& up, const SkinnyPlan& down,
                         float* part_up, float* part_down, uint16_t* A, uint16_t* st0, uint16_t* st1, uint16_t* Y,
                         hipStream_t st) {
  hipError_t e = act == ACT_SWIGLU ? partial_launch<2, false>(up, N, X, h, 0, Wa, Wb, h, Fi, part_up, st)
                                   : partial_launch<1, false>(up, N, X, h, 0, Wa, Wa, h, Fi, part_up, st);
  if (e != hipSuccess) return e;
  const int64_t n_act = (int64_t)N * Fi;
  const dim3 ga(act_blocks(n_act)), ba(256);
  if (act == ACT_SWIGLU)
    hipLaunchKernelGGL(skinny_act<ACT_SWIGLU>, ga, ba, 0, st, part_up, up.ks, n_act, A, st0, st1);
  else if (act == ACT_RELU)
    hipLaunchKernelGGL(skinny_act<ACT_RELU>, ga, ba, 0, st, part_up, up.ks, n_act, A, st0, nullptr);
  else
    hipLaunchKernelGGL(skinny_act<ACT_GELU>, ga, ba, 0, st, part_up, up.ks, n_act, A, st0, nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = partial_launch<1, false>(down, N, A, Fi, 0, W2, W2, Fi, h, part_down, st);
  if (e != hipSuccess) return e;
  return ksum_launch(part_down, down.ks, (int64_t)N * h, Y, st);
}

hipError_t skinny_dgrad_act_launch(int act, int N, const uint16_t* dY, const uint16_t* W2, int h, int Fi,
                                   const SkinnyPlan& p, float* part, const uint16_t* U, const uint16_t* G,
                                   uint16_t* dU, hipStream_t st) {
  hipError_t e = partial_launch<1, true>(p, N, dY, h, 0, W2, W2, h, Fi, part, st);
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)N * Fi;
  const dim3 ga(act_blocks(n)), ba(256);
  if (act == ACT_SWIGLU)
    hipLaunchKernelGGL(skinny_act_bwd<ACT_SWIGLU>, ga, ba, 0, st, part, p.ks, n, Fi, U, G, dU);
  else if (act == ACT_RELU)
    hipLaunchKernelGGL(skinny_act_bwd<ACT_RELU>, ga, ba, 0, st, part, p.ks, n, Fi, U, nullptr, dU);
  else
    hipLaunchKernelGGL(skinny_act_bwd<ACT_GELU>, ga, ba, 0, st, part, p.ks, n, Fi, U, nullptr, dU);
  return hipGetLastError();
}

hipError_t skinny_dgrad_up_launch(int act, int N, const uint16_t* dU, const uint16_t* W1, const uint16_t* Wg, int h,
                                  int Fi, const SkinnyPlan& p, float* part, uint16_t* dX, hipStream_t st) {
  const bool sw = act == ACT_SWIGLU;
  const hipError_t e = sw ? partial_launch<2, true>(p, N, dU, 2 * (int64_t)Fi, Fi, Wg, W1, Fi, h, part, st)
                          : partial_launch<1, true>(p, N, dU, Fi, 0, W1, W1, Fi, h, part, st);
  if (e != hipSuccess) return e;
  return ksum_launch(part, p.ks * (sw ? 2 : 1), (int64_t)N * h, dX, st);
}

hipError_t skinny_product_launch(int N, const uint16_t* X, const uint16_t* W, int K, int ncols, const SkinnyPlan& p,
                                 float* part, uint16_t* Y, hipStream_t st, bool w_nt) {
  const hipError_t e = w_nt ? partial_launch<1, true>(p, N, X, K, 0, W, W, K, ncols, part, st)
                            : partial_launch<1, false>(p, N, X, K, 0, W, W, K, ncols, part, st);
  if (e != hipSuccess) return e;
  return ksum_launch(part, p.ks, (int64_t)N * ncols, Y, st);
}

}  // namespace tpmlp
