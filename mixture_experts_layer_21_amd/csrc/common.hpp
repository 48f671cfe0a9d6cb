// Device helpers shared by the gfx950 kernels of the MoE-layer forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_WAVE 64

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ conversions --

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
  }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) {
    p[i] = f32_to_bf16_bits(v);
  }
};

// ------------------------------------------------------ wave64 reductions --

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, MOE_WAVE));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

// SiLU in fp32: g * 1/(1 + e^-g) with the hardware reciprocal (1 ulp) in
// place of a correctly rounded division (about ten instructions), since the
// result is rounded to the activation dtype or feeds an fp32 product whose
// own rounding is larger; e^-g = inf for large negative g gives -0 as the
// division would.
__device__ __forceinline__ float sigmoid_f32(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
__device__ __forceinline__ float silu_f32(float g) { return g * sigmoid_f32(g); }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (MOE_WAVE - 1); }

// Bits set for lanes strictly below this one.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}
