// Internal interface of the decode GEMV (gemv.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

constexpr int GV_MAX_KR = 2048;  // rows of one k-split (LDS copy of x)

enum GemvEpi : int {
  GV_EPI_STORE = 0,  // out = bf16(sum)
  GV_EPI_ACT = 1,    // out = bf16(act(sum)), st0 = bf16(sum) stash or NULL
  GV_EPI_SWIGLU = 2  // W0 = gate, W1 = up: out = bf16(SiLU(g) * u), st0 = gate, st1 = up stash or NULL
};

struct GemvPlan {
  int strips, ks, kr;
  size_t part_floats;
};

GemvPlan gemv_plan(int K, int ncols, int nmat, int num_cu);

// part: p.part_floats floats; counters: p.strips zero-initialised unsigned
// (left zero on exit).
hipError_t gemv_launch(int epi, int act, const uint16_t* x, const uint16_t* W0, const uint16_t* W1, int K,
                       int ncols, const GemvPlan& p, float* part, unsigned* counters, uint16_t* out,
                       uint16_t* st0, uint16_t* st1, hipStream_t st);

}  // namespace tpmlp
