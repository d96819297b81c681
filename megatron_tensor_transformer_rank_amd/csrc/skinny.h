// Internal interface of the small-batch decode path (skinny.hip): a forward
// for 2 <= N <= SK_MAX_N tokens that streams each weight once, like the
// one-token GEMVs, but multiplies on MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

constexpr int SK_MAX_N = 128;  // largest token count of the small-batch path

struct SkinnyPlan {
  int rows;       // token rows padded to the MFMA tile (16, 32, 64 or 128)
  int strips;     // 256-column strips of one weight matrix
  int ks, kt;     // k-splits, 64-deep k-tiles per split
  size_t part_floats;
  int rtiles;     // row tiles of `rows` rows each (the grid's second dimension)
};

// Split-K plan for X [N, K] @ W [K, ncols] over nmat matrices side by side,
// aiming at target_blocks blocks with at most max_ks k-splits (and at most
// K / (2N), which keeps the float32 partials within the weight's bytes);
// when that leaves the grid at half the target or less, the rows are split
// into tiles as well.  The partials' layout does not depend on the tiles.
SkinnyPlan skinny_plan(int N, int K, int ncols, int nmat, int target_blocks, int max_ks);

// Small-batch forward of one rank's shard: A = act(X @ [Wa, Wb]) (SwiGLU: Wa
// = gate, Wb = up; otherwise Wa = W1, Wb unused), Y = A @ W2.  part_up /
// part_down hold up.part_floats / down.part_floats floats of scratch (no
// initial contents needed).  st0 / st1: stashes or NULL (SwiGLU: gate, up;
// otherwise st0 = U).
hipError_t skinny_launch(int act, int N, const uint16_t* X, const uint16_t* Wa, const uint16_t* Wb,
                         const uint16_t* W2, int h, int Fi, const SkinnyPlan& up, const SkinnyPlan& down,
                         float* part_up, float* part_down, uint16_t* A, uint16_t* st0, uint16_t* st1, uint16_t* Y,
                         hipStream_t st);

// Small-batch backward, input gradients (1 <= N <= SK_MAX_N), with the
// weights read k-contiguous (W2_i [F_i, h] and W1_i, Wg_i [h, F_i] as
// stored):
//   dgrad_act: dA = dY @ W2^T as split-K partials (plan from
//     skinny_plan(N, h, F_i, 1, ...)), then dU = dA * act'(U) (SwiGLU:
//     [dG | dP] from G, U), bf16.
//   dgrad_up:  dX = dU @ W1^T (SwiGLU: dG @ Wg^T + dP @ W1^T, the two k
//     segments as matrices 0 and 1 of the plan skinny_plan(N, F_i, h, 2,
//     ...)), the partials summed with one rounding.
// part holds p.part_floats floats (no initial contents needed).
hipError_t skinny_dgrad_act_launch(int act, int N, const uint16_t* dY, const uint16_t* W2, int h, int Fi,
                                   const SkinnyPlan& p, float* part, const uint16_t* U, const uint16_t* G,
                                   uint16_t* dU, hipStream_t st);
hipError_t skinny_dgrad_up_launch(int act, int N, const uint16_t* dU, const uint16_t* W1, const uint16_t* Wg, int h,
                                  int Fi, const SkinnyPlan& p, float* part, uint16_t* dX, hipStream_t st);

// Y [N, ncols] (bf16) = X [N, K] @ W [K, ncols] (w_nt: @ W^T with W stored
// [ncols, K]) for 1 <= N <= SK_MAX_N: split-K partials (plan p from
// skinny_plan(N, K, ncols, 1, ...)), then their sum in k-split order with one
// rounding.  part holds p.part_floats floats.
hipError_t skinny_product_launch(int N, const uint16_t* X, const uint16_t* W, int K, int ncols, const SkinnyPlan& p,
                                 float* part, uint16_t* Y, hipStream_t st, bool w_nt = false);

}  // namespace tpmlp
