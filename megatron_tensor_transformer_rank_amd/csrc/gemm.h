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
  EPI_ACT_BWD = 4,          // c0 = acc * act'(e0), e0 = pre-activation stash [M, ldc]
  EPI_SWIGLU_BWD = 5        // c0 row = [dG | dP] (ldc = 2*lde); e0 = gate, e1 = up stash (ld = lde)
};

enum GemmKind : int {
  GEMM_UP_ACT = 0,     // X @ W1_i + ReLU/GeLU
  GEMM_UP_SWIGLU = 1,  // X @ [Wg_i, W1_i] + SwiGLU, N = F_i features
  GEMM_DOWN = 2,       // A_i @ W2_i
  GEMM_DGRAD_ACT = 3,  // dY @ W2_i^T with the activation derivative
  GEMM_WGRAD = 4,      // A^T @ B, both operands contiguous along m / n, fp32 out
  GEMM_DGRAD = 5       // dU @ W^T (B read [n][k], optionally two buffers along k)
};

struct GemmArgs {
  int M, N, K;
  // A operand: k-contiguous [m][k] (lda) with an optional split along k into
  // a0 / a1, or m-contiguous [k][m] (lda) for the weight gradients.
  const uint16_t* a0;
  const uint16_t* a1;
  int64_t lda;
  int a_ksplit;
  // B operand: k-contiguous [n][k] (ldb, optional k split into b0 / b1) or
  // n-contiguous [k][n] (ldb); for the SwiGLU forward b0 = gate, b1 = up.
  const uint16_t* b0;
  const uint16_t* b1;
  int64_t ldb;
  int b_ksplit;
  // outputs / epilogue operands
  void* c0;
  void* c1;
  int64_t ldc;
  int c_split;
  void* e0;
  void* e1;
  int64_t lde;
  // filled by the launcher
  int tiles_m, tiles_n;
};

hipError_t gemm_launch(GemmKind kind, int act, const GemmArgs& g, int num_cu, hipStream_t st);

}  // namespace tpmlp
