// Internal interface of the MFMA GEMM (gemm.hip) used by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

enum Epi : int {
  EPI_STORE_BF16 = 0,       // c0 bf16 [M, ldc]
  EPI_STORE_F32_SPLIT = 1,  // fp32; columns < c_split -> c0, the rest -> c1 (col - c_split), both ld = ldc
  EPI_ACT_FWD = 2,          // c0 = act(acc) bf16; e0 (or NULL) = acc bf16 (pre-activation stash)
  EPI_SWIGLU_FWD = 3,       // c0 = SiLU(gate) * up; e0 = gate stash, e1 = up stash (or NULL)
  EPI_ACT_BWD = 4,          // c0 = acc * act'(e0), e0 = pre-activation stash [M, lde]
  EPI_SWIGLU_BWD = 5,       // c0 row = [dG | dP] (ldc = 2*lde); e0 = gate, e1 = up stash (ld = lde)
  EPI_STORE_F32_SLICES = 6  // k-split: fp32 partial of slice s at c0 + s*c_slice, [M, ldc]
};

enum GemmKind : int {
  GEMM_UP_ACT = 0,     // X @ W1_i + ReLU/GeLU
  GEMM_UP_SWIGLU = 1,  // X @ [Wg_i, W1_i] + SwiGLU, N = F_i features
  GEMM_DOWN = 2,       // A_i @ W2_i
  GEMM_DGRAD_ACT = 3,  // dY @ W2_i^T with the activation derivative
  GEMM_WGRAD = 4,      // A^T @ B, both operands contiguous along m / n, fp32 out
  GEMM_DGRAD = 5,      // dU @ W^T (B read [n][k]), one or two k segments
  GEMM_NT_SPLITK = 6   // A @ B^T (B read [n][k]), one segment split along k: fp32 partial per slice
};

// The product runs over one or two k segments; segment s pairs A columns
// [a_koff[s], a_koff[s] + K[s]) (k-contiguous A) with B buffer b[s].  Every
// operand buffer is addressed through a buffer resource of its byte size
// (< 4 GiB), which also zero-fills out-of-range tile lanes.
struct GemmArgs {
  int M, N;
  int nseg;
  int K[2];
  // A: k-contiguous [m][k] (lda) or m-contiguous [k][m] (lda)
  const uint16_t* a[2];
  uint32_t a_bytes[2];
  int a_koff[2];
  int64_t lda;
  // B: k-contiguous [n][k] (ldb) or n-contiguous [k][n] (ldb); SwiGLU
  // forward: b[0] = gate, b[1] = up, one segment
  const uint16_t* b[2];
  uint32_t b_bytes[2];
  int64_t ldb;
  // outputs / epilogue operands
  void* c0;
  void* c1;
  int64_t ldc;
  int c_split;
  void* e0;
  void* e1;
  int64_t lde;
  // split along k (GEMM_NT_SPLITK only: one segment, EPI_STORE_F32_SLICES):
  // slice s of a tile covers k in [s*kslice, min(K[0], (s+1)*kslice)),
  // kslice a multiple of 64, and stores its partial at c0 + s*c_slice
  // floats.  kslice = 0: no split.
  int kslice;
  int64_t c_slice;
  // filled by the launcher
  int tiles_m, tiles_n, ksplit;
};

// Largest operand buffer a GEMM accepts (bytes): buffer resources are 32-bit.
constexpr uint64_t GEMM_MAX_OPERAND_BYTES = 0xFFFFFF00ull;

hipError_t gemm_launch(GemmKind kind, int act, const GemmArgs& g, int num_cu, hipStream_t st);
// Two problems of the same kind and activation in one launch (one tile
// shape, chosen for both): their tiles share the waves, so the partial last
// wave of each is filled by the other's.
hipError_t gemm_launch2(GemmKind kind, int act, const GemmArgs& g0, const GemmArgs& g1, int num_cu, hipStream_t st);

// An input gradient (kind kp: GEMM_DGRAD_ACT with activation act, or
// GEMM_DGRAD) and weight gradients (GEMM_WGRAD: q0, and q1 unless NULL) in
// one launch of 256x256 tiles: the problem with longer tiles is dispatched
// first on every XCD and the other fills in behind it.  Each output element
// is summed over k in the same order as in the separate launches.
hipError_t gemm_launch_mixed(GemmKind kp, int act, const GemmArgs& p, const GemmArgs& q0, const GemmArgs* q1,
                             hipStream_t st);

}  // namespace tpmlp
