// Device-side helpers shared by the HIP kernels of the Domino shard library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace domino {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 <-> fp32. A bf16 value is the top half of an fp32; conversion to bf16 rounds to
// nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element type traits for the generic (fp32 / bf16) paths.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = uint16_t(f32_to_bf16_bits(v)); }
};

// Activations, written from their definitions. σ(x) = 1 / (1 + e^(−x)); the tanh-form
// GeLU uses 0.5·(1 + tanh(u)) = σ(2u) with u = √(2/π)·(x + 0.044715·x³).
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

__device__ __forceinline__ float gelu_tanh_f(float x) {
  const float k0 = 0.7978845608028654f;  // √(2/π)
  const float u = k0 * (x + 0.044715f * x * x * x);
  return x * sigmoidf_(2.0f * u);
}

__device__ __forceinline__ float gelu_tanh_grad_f(float x) {
  const float k0 = 0.7978845608028654f;
  const float u = k0 * (x + 0.044715f * x * x * x);
  const float t = 2.0f * sigmoidf_(2.0f * u) - 1.0f;  // tanh(u)
  const float du = k0 * (1.0f + 3.0f * 0.044715f * x * x);
  return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * du;
}

__device__ __forceinline__ float silu_f(float x) { return x * sigmoidf_(x); }

}  // namespace domino
