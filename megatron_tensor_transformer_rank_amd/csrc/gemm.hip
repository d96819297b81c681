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
//   dgrad W1      A = dU [N,gF_i] (k-contiguous)  B = Wg_i, then W1_i, read as [n=h][k]
//                 (two k segments: [dG | dP] against [Wg_i | W1_i])
//
// Design (MI355X-first):
//  * 256 threads = 4 wave64s in a 2x2 grid; block tile BM x BN x 64, each wave
//    owns (BM/2) x (BN/2) of the output in accumulator registers.
//  * Tiles move HBM -> LDS with buffer-load-to-LDS (16 bytes per lane, no
//    VGPR staging, no ds_write).  Each operand is addressed through a buffer
//    resource of its own size; tile lanes outside the matrix get an offset past
//    the end, for which the buffer unit returns zeros, so ragged tails need no
//    other masking.
//  * LDS layouts (16-byte chunks XOR-swizzled against bank conflicts):
//      k-contiguous operand [row][64 k]: chunk c of row r at slot c ^ (r & 7),
//        fragments read with ds_read_b128;
//      m/n-contiguous operand [64 k][R]: chunk c of k-row r at c ^ 2(r & 3),
//        fragments read with ds_read_b64_tr_b16 (the LDS transpose read), two
//        per 8-k fragment.
//  * Two LDS stages.  Per k-tile: step-1 fragments are read while the step-0
//    MFMAs run; one barrier; the DMA of the tile after next is issued into the
//    stage just released and the next tile's step-0 fragments are read while
//    the step-1 MFMAs run.  DMA has a whole k-tile to land.
//  * The MFMA takes the operands swapped (B fragment first) so each lane holds
//    4 consecutive output columns: 8-byte bf16 / 16-byte fp32 stores.
//  * Block ids are remapped so consecutive tiles land on one XCD (blocks are
//    dispatched round-robin over the 8 XCDs), then grouped GROUP_M tiles along
//    M so the tiles an XCD runs together share operand panels in its L2.
//  * Epilogues: plain bf16 / fp32 store (column split into two buffers),
//    ReLU / GeLU with the pre-activation stash, SwiGLU with gate and up
//    accumulated in the same wave (separate gate / up LDS regions), and the
//    activation derivative reading the stash.
#include "common.h"
#include "gemm.h"

namespace tpmlp {

constexpr int BK = 64;
constexpr int NT = 256;
constexpr int GROUP_M = 4;
constexpr uint32_t OOB = 0xFFFFFFF0u;         // past the end of any accepted buffer
constexpr int RSRC_FLAGS = 0x00020000;        // raw buffer, 32-bit data

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, RSRC_FLAGS);
}
__device__ __forceinline__ void dma16(rsrc_t r, uint8_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, voff, 0, 0, 0);
}
// s_waitcnt with only the vector-memory counter constrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------
// DMA of a k-contiguous operand tile: R rows x 64 k into [row][8 chunks].
// One wave instruction fills 1 KiB = 8 rows; lane i of segment sg holds the
// LDS chunk q = sg*64 + i: row q/8, slot q%8, logical chunk slot ^ (row&7).
// ---------------------------------------------------------------------------
template <int R>
struct DmaK {
  static constexpr int NI = R / 32;  // instructions per wave per tile
  uint32_t voff[NI];                 // row*ld*2 + chunk*16 (bytes from the tile's k0), or OOB
  int kc[NI];                        // element offset of the lane's chunk in the tile
  __device__ __forceinline__ void init(int row0, int rows, int64_t ld, int lane, int w) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = (w + 4 * j) * 64 + lane;
      const int r = q >> 3;
      const int chunk = (q & 7) ^ (r & 7);
      const int grow = row0 + r;
      kc[j] = chunk * 8;
      voff[j] = grow < rows ? (uint32_t)((int64_t)grow * ld * 2) + (uint32_t)kc[j] * 2u : OOB;
    }
  }
  // instruction J of a tile; rs addresses the operand from the tile's first
  // k; chunks at or past kvalid (elements from the tile's first k) read zeros
  template <int J>
  __device__ __forceinline__ void issue(rsrc_t rs, uint8_t* region, int kvalid, int w) const {
    dma16(rs, region + (w + 4 * J) * 1024, kc[J] < kvalid ? voff[J] : OOB);
  }
};

// ---------------------------------------------------------------------------
// DMA of an m/n-contiguous operand tile: 64 k-rows x RW columns into
// [k][RW/8 chunks]; chunk c of k-row r at slot c ^ 2(r&3).
// ---------------------------------------------------------------------------
template <int RW>
struct DmaMN {
  static constexpr int CPR = RW / 8;
  static constexpr int NI = RW / 32;
  uint32_t voff[NI];  // krow*ld*2 + col*2 (bytes from the tile's first k row), or OOB
  __device__ __forceinline__ void init(int col0, int cols, int64_t ld, int lane, int w) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = (w + 4 * j) * 64 + lane;
      const int kr = q / CPR;
      const int chunk = (q % CPR) ^ (2 * (kr & 3));
      const int col = col0 + chunk * 8;
      voff[j] = col < cols ? (uint32_t)((int64_t)kr * ld * 2) + (uint32_t)col * 2u : OOB;
    }
  }
  // instruction J of a tile; rs addresses the operand from the tile's first k
  // row and ends with the operand, so k rows past the end read zeros
  template <int J>
  __device__ __forceinline__ void issue(rsrc_t rs, uint8_t* region, int w) const {
    dma16(rs, region + (w + 4 * J) * 1024, voff[J]);
  }
};

// ---------------------------------------------------------------------------
// Fragment reads (16 rows/columns x 32 k of one MFMA operand, 8 bf16 per lane:
// lane l holds index l%16, k = 8*(l/16) .. +7 of the k-step).
// ---------------------------------------------------------------------------
// k-contiguous region: byte offset of lane's fragment for block row base rb,
// k-step s; block i adds i*2048.
__device__ __forceinline__ int kfrag_off(int rb, int s, int lane) {
  const int l16 = lane & 15, lq = lane >> 4;
  return (rb + l16) * 128 + (((s * 4 + lq) ^ (l16 & 7)) << 4);
}

// m/n-contiguous region of width RW: per-lane k-row byte base and the column
// part of block i (columns cb + 16 i .. +15).
template <int RW>
__device__ __forceinline__ int mn_kbase(int lane) {
  const int g = lane >> 4, src = lane & 15;
  return (8 * g + (src >> 2)) * (RW * 2);
}
__device__ __forceinline__ int mn_coloff(int cb, int i, int lane) {
  const int src = lane & 15;
  const int chunk = (cb + 16 * i + 4 * (src & 3)) >> 3;
  return ((chunk ^ (2 * (src >> 2))) << 4) + (src & 1) * 8;
}
// The k loop is hand-scheduled: LDS reads and MFMAs are volatile inline asm,
// so they issue in source order, interleaved one memory operation per MFMA.
// (The compiler's own schedule issued the next tile's DMA and fragment reads
// in a block between the barrier and the MFMAs, idling the MFMA pipe, and the
// intrinsic form of the transpose read carries no alias information, which
// makes the compiler wait for all in-flight buffer-to-LDS loads before it.)
// LDS read results are consumed only after an explicit lgkmcnt(0) wait.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
template <int OFF>
__device__ __forceinline__ bf16x8 ld_b128(uint32_t addr) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF>
__device__ __forceinline__ v4i16 tr16(uint32_t addr) {
  v4i16 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF) : "memory");
  return r;
}
template <int OFF0, int OFF1>
__device__ __forceinline__ bf16x8 ld_tr2(uint32_t addr) {
  const v4i16 lo = tr16<OFF0>(addr);
  const v4i16 hi = tr16<OFF1>(addr);
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

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
  constexpr int QW = BN / 4;  // SwiGLU: features per wave column
  static_assert(BKD != 2 || (BN == 128 || BN == 256), "SwiGLU tile width");
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w >> 1, wn = w & 1;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = (BKD == 2) ? tn * (BN / 2) : tn * BN;

  // ---- operand buffers per k segment (the buffer resources are built where
  // they are used: captured by reference they would be demoted to scratch)
  const int nseg = g.nseg;
  const uint16_t* const a0p = g.a[0];
  const uint16_t* const b0p = g.b[0];
  const uint16_t* const a1p = (nseg > 1 || BKD == 2) ? g.a[1] : g.a[0];
  const uint16_t* const b1p = (nseg > 1 || BKD == 2) ? g.b[1] : g.b[0];
  const uint32_t a0n = g.a_bytes[0], b0n = g.b_bytes[0];
  const uint32_t a1n = (nseg > 1 || BKD == 2) ? g.a_bytes[1] : g.a_bytes[0];
  const uint32_t b1n = (nseg > 1 || BKD == 2) ? g.b_bytes[1] : g.b_bytes[0];
  const int K0 = g.K[0], K1 = nseg > 1 ? g.K[1] : 0;
  const int ako0 = g.a_koff[0], ako1 = g.a_koff[1];

  // ---- DMA descriptors
  typename std::conditional<AK == 0, DmaK<BM>, DmaMN<BM>>::type da;
  typename std::conditional<BKD == 0, DmaK<BN>, DmaMN<(BKD == 2 ? BN / 2 : BN)>>::type db;
  da.init(m0, g.M, g.lda, lane, w);
  db.init(n0, g.N, g.ldb, lane, w);  // SwiGLU: gate and up shards share columns and layout
  const uint32_t lda2 = (uint32_t)(g.lda * 2), ldb2 = (uint32_t)(g.ldb * 2);

  const int nk0 = (K0 + BK - 1) / BK;
  const int nk = nk0 + (nseg > 1 ? (K1 + BK - 1) / BK : 0);

  constexpr int NIA = BM / 32;             // DMA instructions per wave per tile: A
  constexpr int NIB = BN / 32;             // and B
  constexpr int NI_TILE = NIA + NIB;
  // Per-tile DMA state: buffer resources that start at the tile's first k
  // (k-contiguous: column ko + k0 of every row; m/n-contiguous: row k0) and
  // end with the operand.  Tiles at or past nk get empty resources (every
  // lane reads zeros into a stage nobody reads again), so the loop needs no
  // branches.
  struct TileDma {
    rsrc_t ra, rb, rb2;
    int kvalid;  // valid k elements of the tile (k-contiguous masking)
  };
  // (readfirstlane keeps the descriptor in SGPRs: the values are uniform, but
  // a descriptor the compiler believes divergent is issued in a waterfall loop)
  auto shifted = [](const uint16_t* p, uint32_t bytes, uint32_t skip) __attribute__((always_inline)) {
    const uint64_t a = reinterpret_cast<uint64_t>(p) + skip;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(skip < bytes ? bytes - skip : 0u);
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
  };
  auto tile_dma = [&](int t) __attribute__((always_inline)) {
    TileDma d;
    const bool s1 = t >= nk0;
    const int k0 = (s1 ? t - nk0 : t) * BK;
    const int Ks = s1 ? K1 : K0;
    const bool live = k0 < Ks;
    d.kvalid = live ? Ks - k0 : 0;
    const uint16_t* ap = s1 ? a1p : a0p;
    const uint32_t an = live ? (s1 ? a1n : a0n) : 0u;
    const uint16_t* bp = s1 ? b1p : b0p;
    const uint32_t bn = live ? (s1 ? b1n : b0n) : 0u;
    if constexpr (AK == 0) d.ra = shifted(ap, an, (uint32_t)((s1 ? ako1 : ako0) + k0) * 2u);
    else d.ra = shifted(ap, an, (uint32_t)k0 * lda2);
    if constexpr (BKD == 0) d.rb = shifted(bp, bn, (uint32_t)k0 * 2u);
    else d.rb = shifted(b0p, live ? b0n : 0u, (uint32_t)k0 * ldb2);
    if constexpr (BKD == 2) d.rb2 = shifted(b1p, live ? b1n : 0u, (uint32_t)k0 * ldb2);
    else d.rb2 = d.rb;
    return d;
  };
  auto dma_op = [&](auto J_, const TileDma& d, uint8_t* st) __attribute__((always_inline)) {
    constexpr int J = decltype(J_)::value;
    if constexpr (J < NIA) {
      if constexpr (AK == 0) da.template issue<J>(d.ra, st, d.kvalid, w);
      else da.template issue<J>(d.ra, st, w);
    } else {
      constexpr int JB = J - NIA;
      if constexpr (BKD == 0) db.template issue<JB>(d.rb, st + A_BYTES, d.kvalid, w);
      else if constexpr (BKD == 1 || JB < NIB / 2) db.template issue<JB % NIB>(d.rb, st + A_BYTES, w);
      else db.template issue<JB - NIB / 2>(d.rb2, st + A_BYTES + B_BYTES / 2, w);
    }
  };

  // ---- fragment addressing (loop invariant)
  uint32_t a_koff_s[2], b_koff_s[2];
  uint32_t a_col[AK == 1 ? TM : 1], b_col[BKD != 0 ? TN : 1];
  uint32_t a_kb = 0, b_kb = 0;
  if constexpr (AK == 0) {
    a_koff_s[0] = kfrag_off(wm * WM, 0, lane);
    a_koff_s[1] = kfrag_off(wm * WM, 1, lane);
  } else {
    a_kb = mn_kbase<BM>(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) a_col[i] = a_kb + mn_coloff(wm * WM, i, lane);
  }
  if constexpr (BKD == 0) {
    b_koff_s[0] = A_BYTES + kfrag_off(wn * WN, 0, lane);
    b_koff_s[1] = A_BYTES + kfrag_off(wn * WN, 1, lane);
  } else if constexpr (BKD == 1) {
    b_kb = A_BYTES + mn_kbase<BN>(lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) b_col[j] = b_kb + mn_coloff(wn * WN, j, lane);
  } else {
    b_kb = A_BYTES + mn_kbase<BN / 2>(lane);
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      b_col[j] = b_kb + mn_coloff(wn * QW, j, lane);
      b_col[j + TN / 2] = b_col[j] + B_BYTES / 2;  // same columns in the up region
    }
  }

  // Read op R (0 <= R < TM + TN) of k-step S from the stage at LDS address sa:
  // A fragment R, then B fragment R - TM.
  constexpr int NRD = TM + TN;
  auto read_op = [&](auto S_, auto R_, uint32_t sa, bf16x8 (&af)[TM], bf16x8 (&bfv)[TN]) __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value, R = decltype(R_)::value;
    if constexpr (R < TM) {
      if constexpr (AK == 0) {
        af[R] = ld_b128<R * 2048>(sa + a_koff_s[S]);
      } else {
        constexpr int RS = BM * 2;  // k-row stride
        af[R] = ld_tr2<S * 32 * RS, S * 32 * RS + 4 * RS>(sa + a_col[R]);
      }
    } else {
      constexpr int J = R - TM;
      if constexpr (BKD == 0) {
        bfv[J] = ld_b128<J * 2048>(sa + b_koff_s[S]);
      } else {
        constexpr int RS = (BKD == 2 ? BN / 2 : BN) * 2;
        bfv[J] = ld_tr2<S * 32 * RS, S * 32 * RS + 4 * RS>(sa + b_col[J]);
      }
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA I of a phase: block (I / TN, I % TN).  Inline asm with the
  // accumulator tied in place ("+a"): with the builtin the register allocator
  // rotates the accumulator tile between AGPRs and VGPRs every k-tile (~3
  // moves per MFMA), which halves the MFMA issue rate.  An accumulator is
  // reused only TM*TN MFMAs later, far beyond the dependent-MFMA latency.
  constexpr int NMF = TM * TN;
  auto mfma_op = [](auto I_, f32x4 (&c)[TM][TN], const bf16x8 (&af)[TM], const bf16x8 (&bfv)[TN]) __attribute__((always_inline)) {
    constexpr int I = decltype(I_)::value;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(c[I / TN][I % TN])
                 : "v"(bfv[I % TN]), "v"(af[I / TN]));
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // First memory op of a phase waits this many MFMAs, so the MFMAs that read
  // the fragment registers of the previous phase have issued.  Ops that do
  // not fit between the MFMAs (small tiles) follow them.
  constexpr int LAG = 2;

  // ---- prologue: tiles 0 and 1 in flight, tile 0 published, its step-0
  // fragments read
  {
    const TileDma d0 = tile_dma(0), d1 = tile_dma(1);
    static_for<NI_TILE>([&](auto J) __attribute__((always_inline)) { dma_op(J, d0, stage0); });
    static_for<NI_TILE>([&](auto J) __attribute__((always_inline)) { dma_op(J, d1, stage1); });
  }
  wait_vmcnt<NI_TILE>();
  __syncthreads();
  bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
  const uint32_t st0 = lds_addr(stage0), st1 = lds_addr(stage1);
  static_for<NRD>([&](auto R) __attribute__((always_inline)) { read_op(S0{}, R, st0, a0, b0); });

  for (int t = 0; t < nk; ++t) {
    const uint32_t cur = (t & 1) ? st1 : st0, nxt = (t & 1) ? st0 : st1;
    uint8_t* cur_p = (t & 1) ? stage1 : stage0;
    const TileDma dn = tile_dma(t + 2);
    // phase A: step-0 MFMAs of tile t; step-1 fragments of tile t read in between
    wait_lgkm0();
    static_for<NMF>([&](auto I) __attribute__((always_inline)) {
      mfma_op(I, acc, a0, b0);
      constexpr int R = decltype(I)::value - LAG;
      if constexpr (R >= 0 && R < NRD) read_op(S1{}, std::integral_constant<int, R>{}, cur, a1, b1);
    });
    static_for<NRD>([&](auto R) __attribute__((always_inline)) {
      if constexpr (decltype(R)::value + LAG >= NMF) read_op(S1{}, R, cur, a1, b1);
    });
    // this wave's DMA of tile t+1 has landed, its reads of stage cur are done;
    // after the barrier, everyone's are
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    // phase B: step-1 MFMAs of tile t; step-0 fragments of tile t+1 read from
    // stage nxt, then the DMA of tile t+2 issued into stage cur
    auto phase_b_op = [&](auto P_) __attribute__((always_inline)) {
      constexpr int P = decltype(P_)::value;
      if constexpr (P < NRD) read_op(S0{}, P_, nxt, a0, b0);
      else dma_op(std::integral_constant<int, P - NRD>{}, dn, cur_p);
    };
    // Reads in MFMA slots 1..NRD; DMA op d after MFMA 1 + 3d (a burst of
    // buffer loads stalls MFMA issue; spread out they cost ~6% less).
    constexpr int DMA_STRIDE = 3;
    static_for<NMF>([&](auto I) __attribute__((always_inline)) {
      mfma_op(I, acc, a1, b1);
      constexpr int Iv = decltype(I)::value;
      if constexpr (Iv >= 1 && Iv - 1 < NRD) phase_b_op(std::integral_constant<int, Iv - 1>{});
      constexpr int D = (Iv - 1) / DMA_STRIDE;
      if constexpr (Iv >= 1 && (Iv - 1) % DMA_STRIDE == 0 && D < NI_TILE)
        phase_b_op(std::integral_constant<int, NRD + D>{});
    });
    static_for<NI_TILE>([&](auto D) __attribute__((always_inline)) {
      if constexpr (1 + decltype(D)::value * DMA_STRIDE >= NMF)
        phase_b_op(std::integral_constant<int, NRD + decltype(D)::value>{});
    });
    static_for<NRD>([&](auto P) __attribute__((always_inline)) {
      if constexpr (decltype(P)::value + 1 >= NMF) phase_b_op(P);
    });
  }
  wait_vmcnt<0>();  // no DMA may land after the block has left
  wait_lgkm0();

  // The compiler cannot see the asm MFMAs: give the last ones time to write
  // their results before the epilogue reads the accumulators.
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" ::: "memory");

  // ------------------------------------------------------------------ epilogue
  // Lane holds C[m][n .. n+3] of block (i, j) with m = m0 + wm*WM + i*16 + l16,
  // n = n0 + wn*WN + j*16 + 4*lq (SwiGLU: feature f = n0 + wn*QW + j*16 + 4*lq).
  const int l16 = lane & 15, lq = lane >> 4;
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
        const int f = n0 + wn * QW + j * 16 + 4 * lq;
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
          const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.e0) + (int64_t)m * g.lde + n);
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

// Pick the block tile that minimises (waves of num_cu blocks) x (cost per
// tile), cost per tile ~ bm*bn / efficiency.  Larger tiles re-read less from
// L2 and LDS per flop; the wave count captures quantisation on the CUs.
TileCfg choose_tile(int M, int N_cols, bool swiglu_fwd, int num_cu) {
  static const TileCfg cands[] = {{256, 256}, {256, 192}, {192, 256}, {256, 128}, {128, 256}, {128, 128}};
  static const double eff[] = {1.0, 0.97, 0.97, 0.90, 0.90, 0.75};
  double best = 1e300;
  TileCfg bc = {256, 256};
  for (int c = 0; c < 6; ++c) {
    const int bm = cands[c].bm, bn = cands[c].bn;
    if (swiglu_fwd && bn == 192) continue;
    const int cols_per_tile = swiglu_fwd ? bn / 2 : bn;
    const int64_t tiles = (int64_t)((M + bm - 1) / bm) * ((N_cols + cols_per_tile - 1) / cols_per_tile);
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
  if constexpr (BKD != 2) {
    if (t.bm == 256 && t.bn == 192) return launch_cfg<256, 192, AK, BKD, EPI, ACT>(g, st);
  }
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
