// Internal helpers shared by the gfx950 kernels of libtpmlp.so: vector
// types, bfloat16 packing with round-to-nearest-even, and the activation
// functions and their derivatives evaluated in float32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum Act : int { ACT_RELU = 0, ACT_GELU = 1, ACT_SWIGLU = 2 };

// ---------------------------------------------------------------------------
// bfloat16 <-> float32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two float32 -> two bfloat16 (lo in bits 0..15), round to nearest, ties to
// even, denormals kept, NaN -> a quiet NaN: one v_cvt_pk_bf16_f32, which
// gives the bits of the integer rounding u + 0x7fff + ((u >> 16) & 1) of the
// float's pattern u for every non-NaN input (checked against it over every
// 8th float32 pattern on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// ---------------------------------------------------------------------------
// Activations (float32).  GeLU is the exact erf form, u * Phi(u).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

// Normal CDF Phi(u) and density phi(u) from one exponential.  For x >= 0,
// erfc(x) = t * P(t) * exp(-x^2) with t = 1 / (1 + 0.46 x) and P the degree-7
// polynomial below, a relative-error fit of erfc(x) exp(x^2) / t made by
// csrc/fit_erfc.py (Lawson's iteratively reweighted least squares, toward the
// minimax fit): at most 7e-7 relative error in exact arithmetic, 1.4e-6
// evaluated in float32 for x <= 4 and 4.6e-6 up to x = 9 (where the float32
// rounding of x^2 dominates).  With x = |u| / sqrt 2, exp(-x^2) = exp(-u^2/2):
// Phi(u) = 0.5 erfc(x) for u < 0 and 1 - 0.5 erfc(x) for u >= 0, and
// phi(u) = exp(-u^2 / 2) / sqrt(2 pi).
constexpr float ERFC_P = 0.46f;
constexpr float ERFC_C[8] = {2.595270587e-01f, 2.595572640e-01f, 2.311818941e-01f, 1.868477535e-01f,
                             5.261067550e-02f, 1.691909637e-01f, -2.266292848e-01f, 6.771435323e-02f};
__device__ __forceinline__ void normal_cdf_pdf(float u, float& cdf, float& pdf) {
  const float x = fabsf(u) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(ERFC_P, x, 1.0f));
  float p = ERFC_C[7];
#pragma unroll
  for (int i = 6; i >= 0; --i) p = fmaf(p, t, ERFC_C[i]);
  const float e = __expf(-0.5f * u * u);
  const float q = 0.5f * (p * t) * e;  // 0.5 erfc(|u| / sqrt 2)
  cdf = u >= 0.0f ? 1.0f - q : q;
  pdf = 0.39894228040143268f * e;
}

__device__ __forceinline__ float gelu_f(float u) {
  float cdf, pdf;
  normal_cdf_pdf(u, cdf, pdf);
  return u * cdf;
}
// d/du [u * Phi(u)] = Phi(u) + u * phi(u)
__device__ __forceinline__ float gelu_grad_f(float u) {
  float cdf, pdf;
  normal_cdf_pdf(u, cdf, pdf);
  return fmaf(u, pdf, cdf);
}

template <int ACT>
__device__ __forceinline__ float act_f(float u) {
  if constexpr (ACT == ACT_RELU) return u > 0.0f ? u : 0.0f;
  else return gelu_f(u);
}
template <int ACT>
__device__ __forceinline__ float act_grad_f(float u) {
  if constexpr (ACT == ACT_RELU) return u > 0.0f ? 1.0f : 0.0f;
  else return gelu_grad_f(u);
}

// SwiGLU: a = SiLU(g) * u
__device__ __forceinline__ float swiglu_f(float g, float u) { return g * sigmoidf_(g) * u; }
// d/dg and d/du of SiLU(g) * u, scaled by da.
__device__ __forceinline__ void swiglu_grad_f(float da, float g, float u, float& dg, float& du) {
  const float s = sigmoidf_(g);
  dg = da * u * s * (1.0f + g * (1.0f - s));
  du = da * g * s;
}

}  // namespace tpmlp
