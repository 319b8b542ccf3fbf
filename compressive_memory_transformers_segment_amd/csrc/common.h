// Device-side helpers shared by the gfx950 kernels of the Infini-attention
// forward library. CDNA4 only: 64-lane wavefronts, MFMA bf16 tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ia {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ELU(x) + 1 with alpha = 1: x + 1 for x > 0, exp(x) otherwise. Always > 0.
// ([HF-repro] "Infini-Attention メカニズム", step Memory Retrieval: ELU + 1.)
__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Widen the two bf16 halves of a 32-bit word.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest even, hardware conversion) and pack.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

// Load scalar element i of a q/k/v tensor of storage type T as fp32.
template <typename T> __device__ __forceinline__ float load_as_f32(const T *p, size_t i);
template <> __device__ __forceinline__ float load_as_f32<float>(const float *p, size_t i) {
  return p[i];
}
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p, size_t i) {
  return bf16_to_f32(p[i]);
}

// Store fp32 value as storage type T (bf16: round to nearest even).
template <typename T> __device__ __forceinline__ void store_from_f32(T *p, size_t i, float x);
template <> __device__ __forceinline__ void store_from_f32<float>(float *p, size_t i, float x) {
  p[i] = x;
}
template <> __device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t *p, size_t i,
                                                                     float x) {
  p[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

}  // namespace ia
