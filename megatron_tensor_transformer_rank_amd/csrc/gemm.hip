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
  uint32_t rowbyte[NI];              // byte offset of the lane's row, or OOB
  int kc[NI];                        // element offset of the lane's chunk in the tile
  __device__ __forceinline__ void init(int row0, int rows, int64_t ld, int lane, int w) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = (w + 4 * j) * 64 + lane;
      const int r = q >> 3;
      const int chunk = (q & 7) ^ (r & 7);
      const int grow = row0 + r;
      rowbyte[j] = grow < rows ? (uint32_t)((int64_t)grow * ld * 2) : OOB;
      kc[j] = chunk * 8;
    }
  }
  // k range of this tile in buffer elements: [kbase, kbase + 64), valid below kend
  __device__ __forceinline__ void issue(rsrc_t rs, uint8_t* region, int kbase, int kend, int w) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int k = kbase + kc[j];
      const uint32_t v = (rowbyte[j] != OOB && k < kend) ? rowbyte[j] + (uint32_t)k * 2u : OOB;
      dma16(rs, region + (w + 4 * j) * 1024, v);
    }
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
  uint32_t colbyte[NI];  // byte offset of the lane's column in a row, or OOB
  int krow[NI];
  __device__ __forceinline__ void init(int col0, int cols, int lane, int w) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int q = (w + 4 * j) * 64 + lane;
      const int kr = q / CPR;
      const int chunk = (q % CPR) ^ (2 * (kr & 3));
      const int col = col0 + chunk * 8;
      colbyte[j] = col < cols ? (uint32_t)col * 2u : OOB;
      krow[j] = kr;
    }
  }
  __device__ __forceinline__ void issue(rsrc_t rs, uint8_t* region, int k0, int K, int64_t ld, int w) const {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int k = k0 + krow[j];
      const uint32_t v = (colbyte[j] != OOB && k < K) ? (uint32_t)k * (uint32_t)(ld * 2) + colbyte[j] : OOB;
      dma16(rs, region + (w + 4 * j) * 1024, v);
    }
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
__device__ __forceinline__ bf16x8 ld_b128(const uint8_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

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
// The LDS transpose read is issued through inline asm: the intrinsic form
// carries no alias information, so the compiler would wait for every
// outstanding buffer-to-LDS load before each one, serialising the DMA latency
// into every k-tile.  Its results are consumed only after settle() (below).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
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
// Wait for every outstanding LDS read and make the fragments depend on that
// wait, so no consumer can be scheduled before the data has arrived.
template <int N>
__device__ __forceinline__ void settle(bf16x8 (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(f[i]));
}

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

  // ---- buffer resources per k segment
  rsrc_t ra0 = make_rsrc(g.a[0], g.a_bytes[0]);
  rsrc_t rb0 = make_rsrc(g.b[0], g.b_bytes[0]);
  rsrc_t ra1 = ra0, rb1 = rb0;
  if (g.nseg > 1 || BKD == 2) {
    ra1 = make_rsrc(g.a[1], g.a_bytes[1]);
    rb1 = make_rsrc(g.b[1], g.b_bytes[1]);
  }

  // ---- DMA descriptors
  typename std::conditional<AK == 0, DmaK<BM>, DmaMN<BM>>::type da;
  typename std::conditional<BKD == 0, DmaK<BN>, DmaMN<(BKD == 2 ? BN / 2 : BN)>>::type db, dbu;
  if constexpr (AK == 0) da.init(m0, g.M, g.lda, lane, w);
  else da.init(m0, g.M, lane, w);
  if constexpr (BKD == 0) db.init(n0, g.N, g.ldb, lane, w);
  else db.init(n0, g.N, lane, w);
  if constexpr (BKD == 2) dbu = db;  // gate and up shards share columns and layout

  const int nk0 = (g.K[0] + BK - 1) / BK;
  const int nk = nk0 + (g.nseg > 1 ? (g.K[1] + BK - 1) / BK : 0);

  auto issue_tile = [&](int t, uint8_t* st) {
    const bool s1 = t >= nk0;
    const int k0 = (s1 ? t - nk0 : t) * BK;
    const int Ks = s1 ? g.K[1] : g.K[0];
    const rsrc_t ra = s1 ? ra1 : ra0;
    const rsrc_t rb = s1 ? rb1 : rb0;
    if constexpr (AK == 0) {
      const int ko = s1 ? g.a_koff[1] : g.a_koff[0];
      da.issue(ra, st, ko + k0, ko + Ks, w);
    } else {
      da.issue(ra, st, k0, Ks, g.lda, w);
    }
    if constexpr (BKD == 0) db.issue(rb, st + A_BYTES, k0, Ks, w);
    else if constexpr (BKD == 1) db.issue(rb, st + A_BYTES, k0, Ks, g.ldb, w);
    else {
      db.issue(rb0, st + A_BYTES, k0, Ks, g.ldb, w);
      dbu.issue(rb1, st + A_BYTES + B_BYTES / 2, k0, Ks, g.ldb, w);
    }
  };
  constexpr int NI_TILE = (BM + BN) / 32;  // DMA instructions per wave per tile

  // ---- fragment addressing (loop invariant)
  int a_koff_s[2], b_koff_s[2];
  uint32_t a_col[AK == 1 ? TM : 1], b_col[BKD != 0 ? TN : 1];
  uint32_t a_kb = 0, b_kb = 0;
  if constexpr (AK == 0) {
    a_koff_s[0] = kfrag_off(wm * WM, 0, lane);
    a_koff_s[1] = kfrag_off(wm * WM, 1, lane);
  } else {
    a_kb = mn_kbase<BM>(lane);
#pragma unroll
    for (int i = 0; i < TM; ++i) a_col[i] = mn_coloff(wm * WM, i, lane);
  }
  if constexpr (BKD == 0) {
    b_koff_s[0] = kfrag_off(wn * WN, 0, lane);
    b_koff_s[1] = kfrag_off(wn * WN, 1, lane);
  } else if constexpr (BKD == 1) {
    b_kb = mn_kbase<BN>(lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) b_col[j] = mn_coloff(wn * WN, j, lane);
  } else {
    b_kb = mn_kbase<BN / 2>(lane);
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      b_col[j] = mn_coloff(wn * QW, j, lane);
      b_col[j + TN / 2] = b_col[j] + B_BYTES / 2;  // same columns in the up region
    }
  }

  // fragments of k-step S of the tile in stage st
  auto read_frags = [&](auto S_, const uint8_t* st, bf16x8 (&af)[TM], bf16x8 (&bfv)[TN]) {
    constexpr int S = decltype(S_)::value;
    if constexpr (AK == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = ld_b128(st + a_koff_s[S] + i * 2048);
    } else {
      constexpr int RS = BM * 2;  // k-row stride
      const uint32_t base = lds_addr(st) + a_kb;
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = ld_tr2<S * 32 * RS, S * 32 * RS + 4 * RS>(base + a_col[i]);
    }
    const uint8_t* sb = st + A_BYTES;
    if constexpr (BKD == 0) {
#pragma unroll
      for (int j = 0; j < TN; ++j) bfv[j] = ld_b128(sb + b_koff_s[S] + j * 2048);
    } else {
      constexpr int RS = (BKD == 2 ? BN / 2 : BN) * 2;
      const uint32_t base = lds_addr(sb) + b_kb;
#pragma unroll
      for (int j = 0; j < TN; ++j) bfv[j] = ld_tr2<S * 32 * RS, S * 32 * RS + 4 * RS>(base + b_col[j]);
    }
  };
  auto settle_frags = [&](bf16x8 (&af)[TM], bf16x8 (&bfv)[TN]) {
    if constexpr (AK == 1) settle(af);
    if constexpr (BKD != 0) settle(bfv);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto mfma_all = [&](const bf16x8 (&af)[TM], const bf16x8 (&bfv)[TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfv[j], af[i], acc[i][j], 0, 0, 0);
  };

  // ---- prologue: tiles 0 and 1 in flight, wait for tile 0
  issue_tile(0, stage0);
  if (nk > 1) {
    issue_tile(1, stage1);
    wait_vmcnt<NI_TILE>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  bf16x8 a0[TM], b0[TN], a1[TM], b1[TN];
  read_frags(S0{}, stage0, a0, b0);

  for (int t = 0; t < nk; ++t) {
    uint8_t* cur = (t & 1) ? stage1 : stage0;
    uint8_t* nxt = (t & 1) ? stage0 : stage1;
    settle_frags(a0, b0);  // read during the previous step-1 MFMAs: free
    read_frags(S1{}, cur, a1, b1);
    mfma_all(a0, b0);
    // keep the phases in this order (the scheduler would otherwise hoist the
    // DMA wait above most of the step-0 MFMAs and sink the DMA issue below
    // the step-1 MFMAs)
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();  // this wave's DMA of tile t+1 has landed
    __syncthreads();  // everyone's has; everyone is done reading stage cur
    settle_frags(a1, b1);
    if (t + 2 < nk) issue_tile(t + 2, cur);
    if (t + 1 < nk) read_frags(S0{}, nxt, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mfma_all(a1, b1);
  }

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
