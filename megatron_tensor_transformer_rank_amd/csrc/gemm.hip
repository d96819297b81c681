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
//  * 512 threads = 8 wave64s, two per SIMD, in two groups of four.  Group G
//    owns rows G*BM/2 .. +BM/2 of the block tile, wave q of a group owns
//    columns q*BN/4 .. +BN/4, accumulated in AGPRs.
//  * Ping-pong: the groups alternate between a compute phase (the 2*TM*TN
//    MFMAs of one 64-deep k-tile, from fragments already in registers) and a
//    memory phase (the next k-tile's fragments LDS -> registers, plus its share
//    of the HBM -> LDS DMA).  A barrier ends every phase, so on each SIMD one
//    wave issues MFMAs while the other one's loads and waits run beside it.
//  * Tiles move HBM -> LDS with buffer-load-to-LDS (16 bytes per lane, no
//    VGPR staging).  Each operand is addressed through a buffer resource of
//    its own size; tile lanes outside the matrix get an offset past the end,
//    for which the buffer unit returns zeros, so ragged tails need no other
//    masking.
//  * Two LDS stages, each [A rows of group 0 | A rows of group 1 | B].  The
//    DMA is split by region so that every region is rewritten only after the
//    group(s) reading it are done and lands two or three phases before use:
//      group 0, memory phase of tile s: B of tile s+1;
//      group 1, memory phase of tile s: group-1 A rows of tile s+1 and
//      group-0 A rows of tile s+2.
//  * LDS layouts (16-byte chunks XOR-swizzled against bank conflicts):
//      k-contiguous operand [row][64 k]: chunk c of row r at slot c ^ (r & 7),
//        fragments read with ds_read_b128;
//      m/n-contiguous operand [64 k][R]: chunk c of k-row r at slot
//        c ^ mn_swz(r) (2(r & 3), and bit 3 of r moving the two 16-lane
//        halves of a read to different bank halves), fragments read with
//        ds_read_b64_tr_b16 (the LDS transpose read), two per 8-k fragment.
//  * The MFMA takes the operands swapped (B fragment first) so each lane holds
//    4 consecutive output columns: 8-byte bf16 / 16-byte fp32 stores.
//  * Block ids are remapped so consecutive tiles land on one XCD (blocks are
//    dispatched round-robin over the 8 XCDs), then grouped GROUP_M tiles along
//    M so the tiles an XCD runs together share operand panels in its L2.
//  * Epilogues: plain bf16 / fp32 store (column split into two buffers),
//    ReLU / GeLU with the pre-activation stash, SwiGLU with gate and up
//    accumulated in the same wave (separate gate / up LDS regions), the
//    activation derivative reading the stash, and fp32 k-slice partials.
//    Group 0's epilogue overlaps group 1's last compute phase.
//  * One launch may carry two problems of the same kind (both weight
//    gradients), their tiles sharing the waves; an NT product whose tile grid
//    leaves most CUs idle may run split along k (each k-slice a repeat of the
//    tile grid, fp32 partials summed afterwards in slice order).
#include "common.h"
#include "gemm.h"
#include "tiles.h"

namespace tpmlp {

constexpr int BK = 64;
constexpr int NT = 512;
constexpr int GROUP_M = 4;
// ---------------------------------------------------------------------------
// Block id -> tile: XCD-contiguous, then grouped along M.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int logical_of(int pid, int nb) {
  const int xcd = pid & 7, local = pid >> 3;
  const int per = nb >> 3, rem = nb & 7;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}
__device__ __forceinline__ void tile_in(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = GROUP_M * tiles_n;
  const int gid = logical / group;
  const int first_m = gid * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = logical - gid * group;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

// One block tile of problem g: logical tile lt of its (XCD-ordered) grid;
// with a k-split, lt also counts the slice (the tile grid repeats once per
// slice).  smem holds the two LDS stages.
template <int BM, int BN, int AK, int BKD, int EPI, int ACT>
__device__ __forceinline__ void gemm_tile(const GemmArgs g, int lt, uint8_t* smem) {
  constexpr int HM = BM / 2;                 // rows per group
  constexpr int QN = BN / 4;                 // B-region columns per wave
  constexpr int TM = HM / 16, TN = QN / 16;  // 16x16 blocks per wave
  constexpr int AH_BYTES = HM * 128;         // one group's A rows x 64 k
  constexpr int B_BYTES = BN * 128;
  constexpr int STAGE = 2 * AH_BYTES + B_BYTES;
  constexpr int QF = BN / 8;                 // SwiGLU: features per wave
  static_assert(BKD != 2 || (BN == 128 || BN == 256), "SwiGLU tile width");
  static_assert(HM % 64 == 0 && QN % 16 == 0, "tile shape");

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = w >> 2, q = w & 3;
  // k-split: the problem's tiles repeat once per slice
  constexpr bool SPLIT = EPI == EPI_STORE_F32_SLICES;
  int slice = 0;
  if constexpr (SPLIT) {
    const int tiles = g.tiles_m * g.tiles_n;
    slice = lt / tiles;
    lt -= slice * tiles;
  }
  int tm, tn;
  tile_in(lt, g.tiles_m, g.tiles_n, tm, tn);
  const int m0 = tm * BM;
  const int n0 = (BKD == 2) ? tn * (BN / 2) : tn * BN;

  const int nseg = g.nseg;
  const int kbase = SPLIT ? slice * g.kslice : 0;                      // first k of the slice
  const int K0 = SPLIT ? min(g.K[0], kbase + g.kslice) : g.K[0];        // end of segment 0's range
  const int K1 = nseg > 1 ? g.K[1] : 0;
  const int nk0 = (K0 - kbase + BK - 1) / BK;
  const int nk = nk0 + (nseg > 1 ? (K1 + BK - 1) / BK : 0);

  // Buffer resource that starts `skip` bytes into an operand and ends with it
  // (readfirstlane keeps it in SGPRs: the values are uniform, but a descriptor
  // the compiler believes divergent is issued in a waterfall loop).
  auto shifted = [](const uint16_t* p, uint32_t bytes, uint32_t skip) __attribute__((always_inline)) {
    const uint64_t a = reinterpret_cast<uint64_t>(p) + skip;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(skip < bytes ? bytes - skip : 0u);
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo), n);
  };
  // k range of tile t: segment, first k within it, valid k count (0 past the end)
  struct KTile {
    bool s1;
    int k0, kvalid;
  };
  auto ktile = [&](int t) __attribute__((always_inline)) {
    KTile r;
    r.s1 = t >= nk0;
    r.k0 = r.s1 ? (t - nk0) * BK : kbase + t * BK;
    const int Ks = r.s1 ? K1 : K0;
    r.kvalid = r.k0 < Ks ? Ks - r.k0 : 0;
    return r;
  };

  // ---- fragment addressing (relative to a stage)
  uint32_t a_koff[2] = {0, 0}, b_koff[2] = {0, 0};
  uint32_t a_col[AK == 1 ? TM : 1], b_col[BKD != 0 ? TN : 1];
  const uint32_t a_region = G * AH_BYTES;
  if constexpr (AK == 0) {
    a_koff[0] = a_region + kfrag_off(0, 0, lane);
    a_koff[1] = a_region + kfrag_off(0, 1, lane);
  } else {
    const uint32_t kb = a_region + mn_kbase<HM>(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) a_col[i] = kb + mn_coloff<HM>(0, i, lane);
  }
  if constexpr (BKD == 0) {
    b_koff[0] = 2 * AH_BYTES + kfrag_off(q * QN, 0, lane);
    b_koff[1] = 2 * AH_BYTES + kfrag_off(q * QN, 1, lane);
  } else if constexpr (BKD == 1) {
    const uint32_t kb = 2 * AH_BYTES + mn_kbase<BN>(lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) b_col[j] = kb + mn_coloff<BN>(q * QN, j, lane);
  } else {
    const uint32_t kb = 2 * AH_BYTES + mn_kbase<BN / 2>(lane);
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      b_col[j] = kb + mn_coloff<BN / 2>(q * QF, j, lane);
      b_col[j + TN / 2] = b_col[j] + B_BYTES / 2;  // same features in the up region
    }
  }

  // All fragments of one k-tile (two k-steps of 32) from the stage at sa.
  bf16x8 af[2][TM], bfr[2][TN];
  auto read_tile = [&](uint32_t sa) __attribute__((always_inline)) {
    static_for<2>([&](auto S_) __attribute__((always_inline)) {
      constexpr int S = decltype(S_)::value;
      static_for<TM>([&](auto I_) __attribute__((always_inline)) {
        constexpr int I = decltype(I_)::value;
        if constexpr (AK == 0) {
          af[S][I] = ld_b128<I * 2048>(sa + a_koff[S]);
        } else {
          constexpr int RS = HM * 2;
          af[S][I] = ld_tr2<S * 32 * RS, S * 32 * RS + 4 * RS>(sa + a_col[I]);
        }
      });
      static_for<TN>([&](auto J_) __attribute__((always_inline)) {
        constexpr int J = decltype(J_)::value;
        if constexpr (BKD == 0) {
          bfr[S][J] = ld_b128<J * 2048>(sa + b_koff[S]);
        } else {
          constexpr int RS = (BKD == 2 ? BN / 2 : BN) * 2;
          bfr[S][J] = ld_tr2<S * 32 * RS, S * 32 * RS + 4 * RS>(sa + b_col[J]);
        }
      });
    });
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The 2*TM*TN MFMAs of one k-tile.  Inline asm with the accumulator tied in
  // place ("+a"): with the builtin the register allocator rotates accumulators
  // between AGPRs and VGPRs.  An accumulator is reused only TM*TN MFMAs later.
  auto mfma_op = [](auto S_, auto I_, f32x4 (&c)[TM][TN], const bf16x8 (&a)[2][TM], const bf16x8 (&b)[2][TN])
      __attribute__((always_inline)) {
    constexpr int S = decltype(S_)::value, I = decltype(I_)::value;
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(c[I / TN][I % TN])
                 : "v"(b[S][I % TN]), "v"(a[S][I / TN]));
  };
  auto compute_tile = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
    static_for<TM * TN>([&](auto I) __attribute__((always_inline)) {
      mfma_op(std::integral_constant<int, 0>{}, I, acc, af, bfr);
    });
    static_for<TM * TN>([&](auto I) __attribute__((always_inline)) {
      mfma_op(std::integral_constant<int, 1>{}, I, acc, af, bfr);
    });
    __builtin_amdgcn_s_setprio(0);
  };

  const uint32_t st0 = lds_addr(smem);
  auto stage_addr = [&](int t) __attribute__((always_inline)) { return st0 + (t & 1) * STAGE; };
  auto stage_ptr = [&](int t) __attribute__((always_inline)) { return smem + (t & 1) * STAGE; };

  if (G == 0) {
    // -------- group 0: rows 0 .. HM-1 of the tile; DMA of B
    typename std::conditional<BKD == 0, DmaK<BN>, DmaMN<(BKD == 2 ? BN / 2 : BN)>>::type db;
    db.init(n0, g.N, g.ldb, lane, q);
    const uint32_t ldb2 = (uint32_t)(g.ldb * 2);
    constexpr int NIB = BN / 32;  // B instructions per wave per tile
    auto issue_b = [&](int t) __attribute__((always_inline)) {
      const KTile kt = ktile(t);
      const bool live = kt.kvalid > 0;
      uint8_t* region = stage_ptr(t) + 2 * AH_BYTES;
      if constexpr (BKD == 0) {
        const rsrc_t rb = shifted(kt.s1 ? g.b[1] : g.b[0], live ? (kt.s1 ? g.b_bytes[1] : g.b_bytes[0]) : 0u,
                                  (uint32_t)kt.k0 * 2u);
        static_for<NIB>([&](auto J) __attribute__((always_inline)) {
          db.template issue<decltype(J)::value>(rb, region, kt.kvalid, q);
        });
      } else if constexpr (BKD == 1) {
        const rsrc_t rb = shifted(g.b[0], live ? g.b_bytes[0] : 0u, (uint32_t)kt.k0 * ldb2);
        static_for<NIB>([&](auto J) __attribute__((always_inline)) {
          db.template issue<decltype(J)::value>(rb, region, q);
        });
      } else {
        const rsrc_t rg = shifted(g.b[0], live ? g.b_bytes[0] : 0u, (uint32_t)kt.k0 * ldb2);
        const rsrc_t ru = shifted(g.b[1], live ? g.b_bytes[1] : 0u, (uint32_t)kt.k0 * ldb2);
        static_for<NIB / 2>([&](auto J) __attribute__((always_inline)) {
          db.template issue<decltype(J)::value>(rg, region, q);
        });
        static_for<NIB / 2>([&](auto J) __attribute__((always_inline)) {
          db.template issue<decltype(J)::value>(ru, region + B_BYTES / 2, q);
        });
      }
    };
    // prologue: B of tile 0 (group 1 loads the A rows of tile 0 and group 0's
    // A rows of tile 1)
    issue_b(0);
    wait_vmcnt<0>();
    barrier();
    for (int s = 0; s < nk; ++s) {
      // memory phase: fragments of tile s, DMA of B of tile s+1
      read_tile(stage_addr(s));
      issue_b(s + 1);
      wait_lgkm0();
      barrier();
      // compute phase: tile s; B of tile s+1 must land before the next memory phase
      compute_tile();
      wait_vmcnt<0>();
      barrier();
    }
  } else {
    // -------- group 1: rows HM .. BM-1 of the tile; DMA of both A halves
    typename std::conditional<AK == 0, DmaK<HM>, DmaMN<HM>>::type dtop, dbot;
    dtop.init(m0, g.M, g.lda, lane, q);
    dbot.init(m0 + HM, g.M, g.lda, lane, q);
    const uint32_t lda2 = (uint32_t)(g.lda * 2);
    constexpr int NIA = HM / 32;  // instructions per wave per half tile
    // A rows of group `half` (0: rows 0..HM-1, 1: rows HM..BM-1) of tile t
    auto issue_a = [&](int t, auto half_) __attribute__((always_inline)) {
      constexpr int HALF = decltype(half_)::value;
      const KTile kt = ktile(t);
      const bool live = kt.kvalid > 0;
      const uint16_t* ap = kt.s1 ? g.a[1] : g.a[0];
      const uint32_t an = live ? (kt.s1 ? g.a_bytes[1] : g.a_bytes[0]) : 0u;
      uint8_t* region = stage_ptr(t) + HALF * AH_BYTES;
      const auto& d = HALF == 0 ? dtop : dbot;
      if constexpr (AK == 0) {
        const rsrc_t ra = shifted(ap, an, (uint32_t)((kt.s1 ? g.a_koff[1] : g.a_koff[0]) + kt.k0) * 2u);
        static_for<NIA>([&](auto J) __attribute__((always_inline)) {
          d.template issue<decltype(J)::value>(ra, region, kt.kvalid, q);
        });
      } else {
        const rsrc_t ra = shifted(ap, an, (uint32_t)kt.k0 * lda2);
        static_for<NIA>([&](auto J) __attribute__((always_inline)) {
          d.template issue<decltype(J)::value>(ra, region, q);
        });
      }
    };
    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    issue_a(0, H1{});
    issue_a(0, H0{});
    issue_a(1, H0{});
    wait_vmcnt<0>();
    barrier();
    barrier();  // group 0's first memory phase
    for (int s = 0; s < nk; ++s) {
      // memory phase: fragments of tile s; DMA of this group's rows of tile
      // s+1 and group 0's rows of tile s+2; group 0's rows of tile s+1 must
      // land before its next memory phase
      read_tile(stage_addr(s));
      issue_a(s + 1, H1{});
      issue_a(s + 2, H0{});
      wait_lgkm0();
      wait_vmcnt<2 * NIA>();
      barrier();
      // compute phase: tile s; this group's rows of tile s+1 must land before
      // its next memory phase
      compute_tile();
      if (s + 1 < nk) {
        wait_vmcnt<NIA>();
        barrier();
      }
    }
  }
  wait_vmcnt<0>();  // no DMA may land after the wave has left
  wait_lgkm0();

  // The compiler cannot see the asm MFMAs: give the last ones time to write
  // their results before the epilogue reads the accumulators.
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 7" ::: "memory");

  // ------------------------------------------------------------------ epilogue
  // Lane holds C[m][n .. n+3] of block (i, j) with m = m0 + G*HM + i*16 + l16,
  // n = n0 + q*QN + j*16 + 4*lq (SwiGLU: feature f = n0 + q*QF + j*16 + 4*lq).
  const int l16 = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int m = m0 + G * HM + i * 16 + l16;
    if (m >= g.M) continue;
    if constexpr (EPI == EPI_STORE_BF16) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + q * QN + j * 16 + 4 * lq;
        if (n < g.N) {
          uint2 v = make_uint2(pack_bf16x2(acc[i][j][0], acc[i][j][1]), pack_bf16x2(acc[i][j][2], acc[i][j][3]));
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.c0) + (int64_t)m * g.ldc + n) = v;
        }
      }
    } else if constexpr (EPI == EPI_STORE_F32_SPLIT) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + q * QN + j * 16 + 4 * lq;
        if (n < g.N) {
          float* dst = n < g.c_split ? static_cast<float*>(g.c0) + (int64_t)m * g.ldc + n
                                     : static_cast<float*>(g.c1) + (int64_t)m * g.ldc + (n - g.c_split);
          *reinterpret_cast<float4*>(dst) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
      }
    } else if constexpr (EPI == EPI_STORE_F32_SLICES) {
      float* part = static_cast<float*>(g.c0) + (int64_t)slice * g.c_slice + (int64_t)m * g.ldc;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + q * QN + j * 16 + 4 * lq;
        if (n < g.N)
          *reinterpret_cast<float4*>(part + n) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
    } else if constexpr (EPI == EPI_ACT_FWD) {
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + q * QN + j * 16 + 4 * lq;
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
        const int f = n0 + q * QF + j * 16 + 4 * lq;
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
        const int n = n0 + q * QN + j * 16 + 4 * lq;
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
        const int n = n0 + q * QN + j * 16 + 4 * lq;
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

template <int BM, int BN>
constexpr int stage_bytes() { return 2 * (BM / 2) * 128 + BN * 128; }

// One launch may run two problems of the same kind (g0's nb0 tiles, then
// g1's): the logical tiles of both are laid out over the XCDs together, so
// neither leaves a partial last wave on its own.  A single problem passes
// g1 = g0 and nb0 = the grid size.
template <int BM, int BN, int AK, int BKD, int EPI, int ACT>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
gemm_kernel(const GemmArgs g0, const GemmArgs g1, int nb0) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * stage_bytes<BM, BN>()];
  const int L = logical_of(blockIdx.x, gridDim.x);
  const bool second = L >= nb0;
  const GemmArgs g = second ? g1 : g0;
  gemm_tile<BM, BN, AK, BKD, EPI, ACT>(g, second ? L - nb0 : L, smem);
}

// Mixed grid: the nf tiles of one problem and the tiles of another (a pair
// of the same kind: gs0's ns0 tiles, then gs1's) share one launch.  Every
// XCD runs its share of the first problem's tiles, then its share of the
// second's: with the longer tiles first (the host orders them), the short
// tiles fill in behind them and even out the CUs' finishing times, and the
// tiles of the two problems end at different times, so their output writes
// do not all fall together.
//
// Blocks are dispatched round-robin over the 8 XCDs: XCD x runs blocks
// pid = x + 8j, j = 0, 1, ..., in order.
__device__ __forceinline__ void mixed_of(int pid, int nf, int nb, bool& first, int& idx) {
  const int x = pid & 7, j = pid >> 3;
  const int fq = nf >> 3, fr = nf & 7;
  const int cnt_f = fq + (x < fr ? 1 : 0);
  const int start_f = x * fq + min(x, fr);
  if (j < cnt_f) {
    first = true;
    idx = start_f + j;
    return;
  }
  const int start_all = x * (nb >> 3) + min(x, nb & 7);  // blocks on XCDs before x
  first = false;
  idx = start_all - start_f + (j - cnt_f);
}

template <int BM, int BN, int AKp, int BKDp, int EPIp, int ACTp, int AKq, int BKDq, int EPIq, int ACTq>
__global__ void __attribute__((amdgpu_flat_work_group_size(NT, NT), amdgpu_waves_per_eu(2, 2)))
gemm_mixed_kernel(const GemmArgs gp, const GemmArgs gq0, const GemmArgs gq1, int np, int nq0, int p_first) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * stage_bytes<BM, BN>()];
  const int nb = gridDim.x;
  bool first;
  int idx;
  mixed_of(blockIdx.x, p_first ? np : nb - np, nb, first, idx);
  if (first == (p_first != 0)) {
    gemm_tile<BM, BN, AKp, BKDp, EPIp, ACTp>(gp, idx, smem);
  } else {
    const bool second = idx >= nq0;
    const GemmArgs g = second ? gq1 : gq0;
    gemm_tile<BM, BN, AKq, BKDq, EPIq, ACTq>(g, second ? idx - nq0 : idx, smem);
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
// tile), cost per tile ~ bm*bn / efficiency.  Larger tiles move fewer bytes
// from L2 per flop, which matters twice on a power-limited chip (the clock
// drops with data movement); the wave count captures quantisation on the CUs.
// The 256x192 weight was fitted to timings of both tiles on the weight-
// gradient, down-projection and up-projection shapes of the 7B-, GPT-3- and
// 70B-class shards; the smaller tiles' weights are estimates.
TileCfg choose_tile(int M, int N_cols, bool swiglu_fwd, int num_cu, int M1 = 0, int N1 = 0) {
  static const TileCfg cands[] = {{256, 256}, {256, 192}, {256, 128}, {128, 256}, {128, 128}};
  static const double eff[] = {1.0, 0.87, 0.72, 0.72, 0.5};
  double best = 1e300;
  TileCfg bc = {256, 256};
  for (int c = 0; c < 5; ++c) {
    const int bm = cands[c].bm, bn = cands[c].bn;
    if (swiglu_fwd && bn == 192) continue;
    const int cols_per_tile = swiglu_fwd ? bn / 2 : bn;
    const int64_t tiles = (int64_t)((M + bm - 1) / bm) * ((N_cols + cols_per_tile - 1) / cols_per_tile) +
                          (int64_t)((M1 + bm - 1) / bm) * ((N1 + cols_per_tile - 1) / cols_per_tile);
    const int64_t waves = (tiles + num_cu - 1) / num_cu;
    const double cost = (double)waves * bm * bn / eff[c];
    if (cost < best * 0.999) {
      best = cost;
      bc = cands[c];
    }
  }
  return bc;
}

// g1 == nullptr: one problem
template <int BM, int BN, int AK, int BKD, int EPI, int ACT>
hipError_t launch_cfg(GemmArgs g0, const GemmArgs* g1p, hipStream_t st) {
  const int cols_per_tile = (BKD == 2) ? BN / 2 : BN;
  auto tiles = [&](GemmArgs& g) {
    g.tiles_m = (g.M + BM - 1) / BM;
    g.tiles_n = (g.N + cols_per_tile - 1) / cols_per_tile;
    g.ksplit = g.kslice > 0 ? (g.K[0] + g.kslice - 1) / g.kslice : 1;
    return (int64_t)g.tiles_m * g.tiles_n * g.ksplit;
  };
  GemmArgs g1 = g1p ? *g1p : g0;
  const int64_t nb0 = tiles(g0);
  const int64_t nb = g1p ? nb0 + tiles(g1) : nb0;
  if (!g1p) g1 = g0;
  if (nb <= 0) return hipSuccess;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, AK, BKD, EPI, ACT>), dim3((unsigned)nb), dim3(NT), 0, st, g0, g1,
                     (int)nb0);
  return hipGetLastError();
}

template <int AK, int BKD, int EPI, int ACT>
hipError_t launch_any(const GemmArgs& g, const GemmArgs* g1, TileCfg t, hipStream_t st) {
  if (t.bm == 256 && t.bn == 256) return launch_cfg<256, 256, AK, BKD, EPI, ACT>(g, g1, st);
  if constexpr (BKD != 2) {
    if (t.bm == 256 && t.bn == 192) return launch_cfg<256, 192, AK, BKD, EPI, ACT>(g, g1, st);
  }
  if (t.bm == 256 && t.bn == 128) return launch_cfg<256, 128, AK, BKD, EPI, ACT>(g, g1, st);
  if (t.bm == 128 && t.bn == 256) return launch_cfg<128, 256, AK, BKD, EPI, ACT>(g, g1, st);
  return launch_cfg<128, 128, AK, BKD, EPI, ACT>(g, g1, st);
}

}  // namespace

namespace {

hipError_t launch_kind(GemmKind kind, int act, const GemmArgs& g, const GemmArgs* g1, TileCfg t, hipStream_t st) {
  switch (kind) {
    case GEMM_UP_ACT:
      return act == ACT_RELU ? launch_any<0, 1, EPI_ACT_FWD, ACT_RELU>(g, g1, t, st)
                             : launch_any<0, 1, EPI_ACT_FWD, ACT_GELU>(g, g1, t, st);
    case GEMM_UP_SWIGLU:
      return launch_any<0, 2, EPI_SWIGLU_FWD, ACT_SWIGLU>(g, g1, t, st);
    case GEMM_DOWN:
      return launch_any<0, 1, EPI_STORE_BF16, 0>(g, g1, t, st);
    case GEMM_DGRAD_ACT:
      if (act == ACT_SWIGLU) return launch_any<0, 0, EPI_SWIGLU_BWD, ACT_SWIGLU>(g, g1, t, st);
      return act == ACT_RELU ? launch_any<0, 0, EPI_ACT_BWD, ACT_RELU>(g, g1, t, st)
                             : launch_any<0, 0, EPI_ACT_BWD, ACT_GELU>(g, g1, t, st);
    case GEMM_WGRAD:
      return launch_any<1, 1, EPI_STORE_F32_SPLIT, 0>(g, g1, t, st);
    case GEMM_DGRAD:
      return launch_any<0, 0, EPI_STORE_BF16, 0>(g, g1, t, st);
    case GEMM_NT_SPLITK:
      return launch_any<0, 0, EPI_STORE_F32_SLICES, 0>(g, g1, t, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm_launch(GemmKind kind, int act, const GemmArgs& g, int num_cu, hipStream_t st) {
  // a k-split repeats the tile grid once per slice: chosen as for M * slices rows
  const int slices = g.kslice > 0 ? (g.K[0] + g.kslice - 1) / g.kslice : 1;
  const TileCfg t = choose_tile(g.M * slices, g.N, kind == GEMM_UP_SWIGLU, num_cu);
  return launch_kind(kind, act, g, nullptr, t, st);
}

hipError_t gemm_launch2(GemmKind kind, int act, const GemmArgs& g0, const GemmArgs& g1, int num_cu, hipStream_t st) {
  const TileCfg t = choose_tile(g0.M, g0.N, kind == GEMM_UP_SWIGLU, num_cu, g1.M, g1.N);
  return launch_kind(kind, act, g0, &g1, t, st);
}

namespace {

int k_tiles(const GemmArgs& g) {
  return (g.K[0] + BK - 1) / BK + (g.nseg > 1 ? (g.K[1] + BK - 1) / BK : 0);
}

template <int BM, int BN, int AKp, int BKDp, int EPIp, int ACTp>
hipError_t launch_mixed_wgrad(GemmArgs p, GemmArgs q0, const GemmArgs* q1p, hipStream_t st) {
  auto tiles = [](GemmArgs& g) {
    g.tiles_m = (g.M + BM - 1) / BM;
    g.tiles_n = (g.N + BN - 1) / BN;
    g.ksplit = 1;
    return (int64_t)g.tiles_m * g.tiles_n;
  };
  GemmArgs q1 = q1p ? *q1p : q0;
  const int64_t np = tiles(p), nq0 = tiles(q0);
  const int64_t nq = q1p ? nq0 + tiles(q1) : nq0;
  if (!q1p) q1 = q0;
  const int64_t nb = np + nq;
  if (nb <= 0) return hipSuccess;
  if (nb > 0x7fffffff) return hipErrorInvalidValue;
  // the problem with more k-tiles per block tile is dispatched first
  const int kq = q1p ? (k_tiles(q0) > k_tiles(q1) ? k_tiles(q0) : k_tiles(q1)) : k_tiles(q0);
  const int p_first = k_tiles(p) >= kq ? 1 : 0;
  hipLaunchKernelGGL((gemm_mixed_kernel<BM, BN, AKp, BKDp, EPIp, ACTp, 1, 1, EPI_STORE_F32_SPLIT, 0>), dim3((unsigned)nb),
                     dim3(NT), 0, st, p, q0, q1, (int)np, (int)nq0, p_first);
  return hipGetLastError();
}

}  // namespace

hipError_t gemm_launch_mixed(GemmKind kp, int act, const GemmArgs& p, const GemmArgs& q0, const GemmArgs* q1,
                             hipStream_t st) {
  if (kp == GEMM_DGRAD) return launch_mixed_wgrad<256, 256, 0, 0, EPI_STORE_BF16, 0>(p, q0, q1, st);
  if (kp != GEMM_DGRAD_ACT) return hipErrorInvalidValue;
  if (act == ACT_SWIGLU) return launch_mixed_wgrad<256, 256, 0, 0, EPI_SWIGLU_BWD, ACT_SWIGLU>(p, q0, q1, st);
  if (act == ACT_RELU) return launch_mixed_wgrad<256, 256, 0, 0, EPI_ACT_BWD, ACT_RELU>(p, q0, q1, st);
  return launch_mixed_wgrad<256, 256, 0, 0, EPI_ACT_BWD, ACT_GELU>(p, q0, q1, st);
}

}  // namespace tpmlp
