// Device helpers shared by the gfx950 kernels of the GPT step.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace gk {

typedef uint16_t bf16;   // raw bf16 bits; arithmetic is always done in fp32

__device__ __forceinline__ float bf2f(bf16 v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16x2 (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack2bf(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)(pack2bf(f, 0.f) & 0xFFFFu); }

// Storage-type load/store (float or bf16 bits).
__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16* p, int64_t i) { return bf2f(p[i]); }
__device__ __forceinline__ void st(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st(bf16* p, int64_t i, float v) { p[i] = f2bf(v); }
// value as it reads back after being stored
__device__ __forceinline__ float rnd_as(const float*, float v) { return v; }
__device__ __forceinline__ float rnd_as(const bf16*, float v) { return bf2f(f2bf(v)); }

// Wavefront (64 lanes) reductions.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// Sum within aligned segments of `seg` lanes (seg a power of two <= 64).
__device__ __forceinline__ float seg_sum(float v, int seg) {
  for (int o = seg >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace gk
