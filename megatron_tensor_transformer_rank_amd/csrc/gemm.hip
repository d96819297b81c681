// bf16 MFMA GEMM for gfx950 with the fused epilogues of the TP MLP shard.
//
// C[M, N] = sum_k A[m, k] * B[k, n], bf16 operands, float32 accumulation on
// v_mfma_f32_16x16x32_bf16.  One kernel template covers the six products of
// one rank's forward and backward ("02 -- Tensor Parallelism", sections
// "Column-parallel", "Row-parallel", "The MLP pairing"; "Parallelism
// Strategies #1 - Tensor Parallelism", sharded backward):
//
//   up + act      A = X [N,h] (k-contiguous)      B = W1_i [h,F_i] (n-contiguous)
//   down          A = A_i [N,F_i] (k-contiguous)  B = W2_i [F_i,h] (n-contiguous)
//   dgrad W2+act' A = dY [N,h] (k-contiguous)     B = W2_i read as [n=F_i][k=h]
//   wgrad W2      A = A_i read as [k=N][m=F_i]    B = dY [k=N][n=h]
//   wgrad W1      A = X read as [k=N][m=h]        B = dU [k=N][n=gF_i]
//   dgrad W1      A = dU [N,gF_i] (k-contiguous)  B = [Wg_i|W1_i] read as [n=h][k]
//
// Design (MI355X-first):
//  * 256 threads = 4 wave64s in a 2x2 grid; block tile BM x BN x 64, each wave
//    owns (BM/2) x (BN/2) of the output in AGPR/VGPR accumulators.
//  * Both operands are staged in LDS as [row = m or n][64 k] bf16, 128 bytes
//    per row, 16-byte chunks XOR-swizzled by the row so that the b128 fragment
//    reads and the b128 stores are bank-conflict free.  Operands that are
//    contiguous along m/n in HBM (the weight matrices in the forward, both
//    operands of the weight gradients) are loaded as 8x8 bf16 blocks with
//    coalesced 16-byte loads and transposed in registers before the LDS store.
//  * Two LDS stages; the next k-tile is fetched from HBM into registers while
//    the current one feeds the MFMAs, one barrier per k-tile.
//  * The MFMA is issued with the operands swapped (B fragment first) so each
//    lane ends up holding 4 consecutive output columns: 8-byte bf16 and
//    16-byte fp32 stores in the epilogue.
//  * Block ids are remapped so consecutive tiles land on one XCD (blocks are
//    dispatched round-robin over the 8 XCDs), then grouped GROUP_M tiles along
//    M so the tiles an XCD runs together share operand panels in its L2.
//  * Epilogues: plain bf16 / fp32 store (with a column split into two output
//    buffers), activation (ReLU / GeLU) with the pre-activation stash, SwiGLU
//    with gate and up accumulated in the same wave (the B tile interleaves the
//    two weight shards), and the activation derivative that reads the stash.
#include "common.h"
#include "gemm.h"

namespace tpmlp {

constexpr int BK = 64;
constexpr int NT = 256;
constexpr int GROUP_M = 4;

// Slot of a 16-byte chunk inside a 128-byte LDS row.  Depends on row mod 16
// only, so fragment addresses of row blocks 16 apart differ by an immediate.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ uint32_t pick_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pick_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ __forceinline__ uint32_t w_of(const uint4& v, int q) {
  return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// Output element i (0..7) of an 8x8 bf16 transpose: the 8 k-values of column i.
__device__ __forceinline__ uint4 transpose_col(const uint4 (&in)[8], int i) {
  const int q = i >> 1;
  uint4 o;
  if (i & 1) {
    o.x = pick_hi(w_of(in[0], q), w_of(in[1], q));
    o.y = pick_hi(w_of(in[2], q), w_of(in[3], q));
    o.z = pick_hi(w_of(in[4], q), w_of(in[5], q));
    o.w = pick_hi(w_of(in[6], q), w_of(in[7], q));
  } else {
    o.x = pick_lo(w_of(in[0], q), w_of(in[1], q));
    o.y = pick_lo(w_of(in[2], q), w_of(in[3], q));
    o.z = pick_lo(w_of(in[4], q), w_of(in[5], q));
    o.w = pick_lo(w_of(in[6], q), w_of(in[7], q));
  }
  return o;
}

// ---------------------------------------------------------------------------
// Operand tile loaders: HBM -> registers (load) and registers -> LDS (store).
// ROWS is the tile extent along m (A) or n (B).
// ---------------------------------------------------------------------------

// Operand stored [row][k], k contiguous; optionally the k range is the
// concatenation of two buffers (k < ksplit from p0, the rest from p1 at
// k - ksplit), both with leading dimension ld.
template <int ROWS>
struct LoadK {
  static constexpr int NL = ROWS / 32;  // 16-byte chunks per thread
  uint4 r[NL];
  __device__ __forceinline__ void load(const uint16_t* p0, const uint16_t* p1, int64_t ld, int ksplit,
                                       int rows, int K, int row0, int k0, int tid) {
    const int c = tid & 7;
    const int gk = k0 + c * 8;
    const bool kok = gk < K;
    const uint16_t* base = gk < ksplit ? p0 + gk : p1 + (gk - ksplit);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int row = row0 + (tid >> 3) + 32 * i;
      if (kok && row < rows)
        r[i] = *reinterpret_cast<const uint4*>(base + (int64_t)row * ld);
      else
        r[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
    const int c = tid & 7;
    const int rr = tid >> 3;
    uint8_t* p = lds + rr * 128 + ((c ^ swz(rr)) << 4);
#pragma unroll
    for (int i = 0; i < NL; ++i) *reinterpret_cast<uint4*>(p + i * 32 * 128) = r[i];
  }
};

// Operand stored [k][col], col contiguous.  Loaded as 8 (k) x 8 (col) blocks;
// block b: k-chunk kc = b % 8, col block cb = b / 8.  MAP = 0: tile column n
// is buffer column col0 + n of p0.  MAP = 1 (SwiGLU up-projection B tile):
// the tile's BN columns are, per half (one wave column), QW gate columns then
// the QW up columns of the same features: n -> (w = n / (2QW), r = n % (2QW)),
// buffer = r < QW ? p0 (gate) : p1 (up), column f0 + w*QW + r % QW.
template <int ROWS, int MAP>
struct LoadMN {
  uint4 r[8];
  bool active;
  __device__ __forceinline__ void load(const uint16_t* p0, const uint16_t* p1, int64_t ld, int cols, int K,
                                       int col0, int k0, int tid) {
    active = tid < ROWS;
    if (!active) return;
    const int kc = tid & 7, cb = tid >> 3;
    const int n = cb * 8;
    const uint16_t* buf;
    int col;
    if constexpr (MAP == 0) {
      buf = p0;
      col = col0 + n;
    } else {
      constexpr int QW = ROWS / 4;
      const int w = n / (2 * QW), rr = n % (2 * QW);
      buf = rr < QW ? p0 : p1;
      col = col0 + w * QW + (rr % QW);
    }
    const bool cok = col < cols;
    const uint16_t* base = buf + col;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + kc * 8 + j;
      if (cok && k < K)
        r[j] = *reinterpret_cast<const uint4*>(base + (int64_t)k * ld);
      else
        r[j] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds, int tid) const {
    if (!active) return;
    const int kc = tid & 7, cb = tid >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = cb * 8 + i;
      *reinterpret_cast<uint4*>(lds + row * 128 + ((kc ^ swz(row)) << 4)) = transpose_col(r, i);
    }
  }
};

// ---------------------------------------------------------------------------
// Block id -> tile: XCD-contiguous, then grouped along M.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tile_of(int pid, int nb, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int xcd = pid & 7, local = pid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int group = GROUP_M * tiles_n;
  const int gid = logical / group;
  const int first_m = gid * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - gid * group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

template <int BM, int BN, int AK, int BKD, int EPI, int ACT>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(1, 1)))
gemm_kernel(const GemmArgs g) {
  constexpr int TM = BM / 32, TN = BN / 32;  // 16x16 blocks per wave
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int A_BYTES = BM * 128, B_BYTES = BN * 128;
  constexpr int STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM;
  // For the SwiGLU forward the tile covers BN/2 features (gate + up).
  const int n0 = (BKD == 2) ? tn * (BN / 2) : tn * BN;

  using ALd = typename std::conditional<AK == 0, LoadK<BM>, LoadMN<BM, 0>>::type;
  using BLd = typename std::conditional<BKD == 0, LoadK<BN>,
              typename std::conditional<BKD == 1, LoadMN<BN, 0>, LoadMN<BN, 1>>::type>::type;
  ALd la;
  BLd lb;

  auto load = [&](int k0) {
    if constexpr (AK == 0) la.load(g.a0, g.a1, g.lda, g.a_ksplit, g.M, g.K, m0, k0, tid);
    else la.load(g.a0, g.a1, g.lda, g.M, g.K, m0, k0, tid);
    if constexpr (BKD == 0) lb.load(g.b0, g.b1, g.ldb, g.b_ksplit, g.N, g.K, n0, k0, tid);
    else lb.load(g.b0, g.b1, g.ldb, g.N, g.K, n0, k0, tid);
  };
  auto store = [&](int stage) {
    la.store(smem + stage * STAGE, tid);
    lb.store(smem + stage * STAGE + A_BYTES, tid);
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int l16 = lane & 15, lq = lane >> 4;
  const int a_row = wm * WM + l16;
  const int b_row = wn * WN + l16;
  const int sw = swz(l16);

  const int nk = (g.K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
    const uint8_t* As = smem + cur * STAGE;
    const uint8_t* Bs = As + A_BYTES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int slot = ((s * 4 + lq) ^ sw) << 4;
      bf16x8 af[TM], bfv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (a_row + i * 16) * 128 + slot);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfv[j] = *reinterpret_cast<const bf16x8*>(Bs + (b_row + j * 16) * 128 + slot);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfv[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store(cur ^ 1);
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  // Lane holds C[m][n .. n+3] of block (i, j) with m = m0 + wm*WM + i*16 + l16,
  // n = n0 + wn*WN + j*16 + 4*lq (SwiGLU: feature f = n0 + wn*WN/2 + j*16 + 4*lq).
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + wm * WM + i * 16 + l16;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_STORE_BF16) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * lq;
        if (n < g.N) {
          uint2 v = make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c0) + (int64_t)m * g.ldc + n) = v;
        }
      }
    } else if constexpr (EPI == EPI_STORE_F32_SPLIT) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * lq;
        if (n < g.N) {
          float* dst = n < g.c_split ? static_cast<float*>(g.c0) + (int64_t)m * g.ldc + n
                                     : static_cast<float*>(g.c1) + (int64_t)m * g.ldc + (n - g.c_split);
          *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    } else if constexpr (EPI == EPI_ACT_FWD) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * lq;
        if (n < g.N) {
          const int64_t off = (int64_t)m * g.ldc + n;
          float a[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) a[r] = act_f<ACT>(acc[i][j][r]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c0) + off) =
              make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
          if (g.e0)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.e0) + off) =
                make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
        }
      }
    } else if constexpr (EPI == EPI_SWIGLU_FWD) {
#pragma unroll
      for (int j = 0; j < TN / 2; ++j) {
        const int f = n0 + wn * (WN / 2) + j * 16 + 4 * lq;
        if (f < g.N) {
          const int64_t off = (int64_t)m * g.ldc + f;
          const f32x4 gt = acc[i][j], up = acc[i][j + TN / 2];
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c0) + off) =
              make_uint2(pack_bf16x2(swiglu_f(gt[0], up[0]), swiglu_f(gt[1], up[1])),
                         pack_bf16x2(swiglu_f(gt[2], up[2]), swiglu_f(gt[3], up[3])));
          if (g.e0)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.e0) + off) =
                make_uint2(pack_bf16x2(gt[0], gt[1]), pack_bf16x2(gt[2], gt[3]));
          if (g.e1)
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.e1) + off) =
                make_uint2(pack_bf16x2(up[0], up[1]), pack_bf16x2(up[2], up[3]));
        }
      }
    } else if constexpr (EPI == EPI_ACT_BWD) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * lq;
        if (n < g.N) {
          const int64_t off = (int64_t)m * g.ldc + n;
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.e0) + off);
          const float uu[4] = {bf16lo(u.x), bf16hi(u.x), bf16lo(u.y), bf16hi(u.y)};
          float d[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) d[r] = acc[i][j][r] * act_grad_f<ACT>(uu[r]);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c0) + off) =
              make_uint2(pack_bf16x2(d[0], d[1]), pack_bf16x2(d[2], d[3]));
        }
      }
    } else {  // EPI_SWIGLU_BWD: dU row is [dG | dP], ldc = 2 * F_i, stashes have ld = lde
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 16 + 4 * lq;
        if (n < g.N) {
          const int64_t so = (int64_t)m * g.lde + n;
          const uint2 gb = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.e0) + so);
          const uint2 ub = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.e1) + so);
          const float gg[4] = {bf16lo(gb.x), bf16hi(gb.x), bf16lo(gb.y), bf16hi(gb.y)};
          const float uu[4] = {bf16lo(ub.x), bf16hi(ub.x), bf16lo(ub.y), bf16hi(ub.y)};
          float dg[4], dp[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) swiglu_grad_f(acc[i][j][r], gg[r], uu[r], dg[r], dp[r]);
          uint16_t* row = static_cast<uint16_t*>(g.c0) + (int64_t)m * g.ldc;
          *reinterpret_cast<uint2*>(row + n) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>(row + g.lde + n) =
              make_uint2(pack_bf16x2(dp[0], dp[1]), pack_bf16x2(dp[2], dp[3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: tile choice and launch.
// ---------------------------------------------------------------------------
namespace {

struct TileCfg {
  int bm, bn;
};

// Pick the block tile that minimises (waves of 256 blocks) x (cost per tile),
// cost per tile ~ bm*bn / efficiency.  Larger tiles re-read less from L2 and
// LDS per flop; the wave count captures quantisation on 256 CUs.
TileCfg choose_tile(int M, int N_tiles_cols, bool swiglu_fwd, int num_cu) {
  static const TileCfg cands[] = {{256, 256}, {256, 192}, {192, 256}, {256, 128}, {128, 256}, {128, 128}};
  static const double eff[] = {1.0, 0.97, 0.97, 0.90, 0.90, 0.75};
  double best = 1e300;
  TileCfg bc = {256, 256};
  for (int c = 0; c < 6; ++c) {
    const int bm = cands[c].bm, bn = cands[c].bn;
    const int cols_per_tile = swiglu_fwd ? bn / 2 : bn;
    const int64_t tiles = (int64_t)((M + bm - 1) / bm) * ((N_tiles_cols + cols_per_tile - 1) / cols_per_tile);
    const int64_t waves = (tiles + num_cu - 1) / num_cu;
    const double cost = (double)waves * bm * bn / eff[c];
    if (cost < best * 0.999) {
      best = cost;
      bc = cands[c];
    }
  }
  return bc;
}

template <int BM, int BN, int AK, int BKD, int EPI, int ACT>
hipError_t launch_cfg(GemmArgs g, hipStream_t st) {
  const int cols_per_tile = (BKD == 2) ? BN / 2 : BN;
  g.tiles_m = (g.M + BM - 1) / BM;
  g.tiles_n = (g.N + cols_per_tile - 1) / cols_per_tile;
  const int64_t nb = (int64_t)g.tiles_m * g.tiles_n;
  if (nb <= 0) return hipSuccess;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKD, EPI, ACT>), dim3((unsigned)nb), dim3(NT), 0, st, g);
  return hipGetLastError();
}

template <int AK, int BKD, int EPI, int ACT>
hipError_t launch_any(const GemmArgs& g, TileCfg t, hipStream_t st) {
  if (t.bm == 256 && t.bn == 256) return launch_cfg<256, 256, AK, BKD, EPI, ACT>(g, st);
  if (t.bm == 256 && t.bn == 192) return launch_cfg<256, 192, AK, BKD, EPI, ACT>(g, st);
  if (t.bm == 192 && t.bn == 256) return launch_cfg<192, 256, AK, BKD, EPI, ACT>(g, st);
  if (t.bm == 256 && t.bn == 128) return launch_cfg<256, 128, AK, BKD, EPI, ACT>(g, st);
  if (t.bm == 128 && t.bn == 256) return launch_cfg<128, 256, AK, BKD, EPI, ACT>(g, st);
  return launch_cfg<128, 128, AK, BKD, EPI, ACT>(g, st);
}

}  // namespace

hipError_t gemm_launch(GemmKind kind, int act, const GemmArgs& g, int num_cu, hipStream_t st) {
  const bool sw = kind == GEMM_UP_SWIGLU;
  const TileCfg t = choose_tile(g.M, g.N, sw, num_cu);
  switch (kind) {
    case GEMM_UP_ACT:
      return act == ACT_RELU ? launch_any<0, 1, EPI_ACT_FWD, ACT_RELU>(g, t, st)
                             : launch_any<0, 1, EPI_ACT_FWD, ACT_GELU>(g, t, st);
    case GEMM_UP_SWIGLU:
      return launch_any<0, 2, EPI_SWIGLU_FWD, ACT_SWIGLU>(g, t, st);
    case GEMM_DOWN:
      return launch_any<0, 1, EPI_STORE_BF16, 0>(g, t, st);
    case GEMM_DGRAD_ACT:
      if (act == ACT_SWIGLU) return launch_any<0, 0, EPI_SWIGLU_BWD, ACT_SWIGLU>(g, t, st);
      return act == ACT_RELU ? launch_any<0, 0, EPI_ACT_BWD, ACT_RELU>(g, t, st)
                             : launch_any<0, 0, EPI_ACT_BWD, ACT_GELU>(g, t, st);
    case GEMM_WGRAD:
      return launch_any<1, 1, EPI_STORE_F32_SPLIT, 0>(g, t, st);
    case GEMM_DGRAD:
      return launch_any<0, 0, EPI_STORE_BF16, 0>(g, t, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
