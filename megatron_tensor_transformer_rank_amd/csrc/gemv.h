// Internal interface of the decode GEMVs (gemv.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

constexpr int GV_MAX_KR = 2048;  // rows of one k-split (LDS copy of x)

// Blocks per GEMV, measured best for the one-token stream on 256 CUs: the
// up-projection ~224 (fewer k-splits leave fewer partials for the
// down-projection's prologue to add), the down-projection ~256 (one per CU).
constexpr int DECODE_UP_BLOCKS = 224;
constexpr int DECODE_DOWN_BLOCKS = 256;

struct GemvPlan {
  int strips, ks, kr;
  size_t part_floats;
};

// Split-K plan for a [K, ncols] weight read by nmat matrices side by side.
GemvPlan gemv_plan(int K, int ncols, int nmat, int target_blocks);

// One-token forward: A = act(x @ [Wa, Wb]) (SwiGLU: Wa = gate, Wb = up;
// otherwise Wa = W1 and Wb unused), Y = A @ W2.  part_up / part_down hold
// up.part_floats / down.part_floats floats and cnt down.strips ints (no
// initial contents needed: the first kernel zeroes cnt for the second).
// st0 / st1: stashes or NULL (SwiGLU: gate, up; otherwise st0 = U).
hipError_t decode_launch(int act, const uint16_t* x, const uint16_t* Wa, const uint16_t* Wb, const uint16_t* W2,
                         int h, int Fi, const GemvPlan& up, const GemvPlan& down, float* part_up, float* part_down,
                         int* cnt, uint16_t* A, uint16_t* st0, uint16_t* st1, uint16_t* Y, hipStream_t st);

// out[c] = bf16(sum_{q<ks} part[q][c]) for c < n (n % 4 == 0), in fixed order.
hipError_t ksum_launch(const float* part, int ks, int64_t n, uint16_t* out, hipStream_t st);

}  // namespace tpmlp
