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

// float32 -> bfloat16 bits, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---------------------------------------------------------------------------
// Activations (float32).  GeLU is the exact erf form.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + __expf(-z)); }

__device__ __forceinline__ float gelu_f(float u) {
  return 0.5f * u * (1.0f + erff(u * 0.70710678118654752f));
}
// d/du [u * Phi(u)] = Phi(u) + u * phi(u)
__device__ __forceinline__ float gelu_grad_f(float u) {
  const float cdf = 0.5f * (1.0f + erff(u * 0.70710678118654752f));
  const float pdf = 0.39894228040143268f * __expf(-0.5f * u * u);
  return cdf + u * pdf;
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
