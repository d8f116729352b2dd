// Device-side helpers shared by the gfx950 kernels of the fused-chain library:
// 16-byte vector access, fp32 <-> fp16/bf16 conversion (round to nearest even,
// the hardware's default mode), and a wave64 sum built on DPP row rotations.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fastmath.h"

namespace np {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element conversions. _Float16 -> v_cvt_f16_f32 / v_cvt_f32_f16; __bf16 ->
// v_cvt_pk_bf16_f32 on gfx950 (both round to nearest even) and an exact shift back.
__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(_Float16 x) { return (float)x; }
__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f(float x);
template <>
__device__ __forceinline__ float from_f<float>(float x) { return x; }
template <>
__device__ __forceinline__ _Float16 from_f<_Float16>(float x) { return (_Float16)x; }
template <>
__device__ __forceinline__ __bf16 from_f<__bf16>(float x) { return (__bf16)x; }

// Round an fp32 value to T and back (a cast node / a stored intermediate).
template <typename T>
__device__ __forceinline__ float round_via(float x) { return to_f(from_f<T>(x)); }

template <typename T>
struct Vec {
  static constexpr int N = 16 / sizeof(T);
};

// 16-byte load of N elements converted to fp32 (global_load_dwordx4).
template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[Vec<T>::N]) {
  u32x4 raw = *reinterpret_cast<const u32x4*>(p);
  T e[Vec<T>::N];
  __builtin_memcpy(e, &raw, 16);
#pragma unroll
  for (int i = 0; i < Vec<T>::N; ++i) v[i] = to_f(e[i]);
}

// 16-byte store of N fp32 values rounded to T (global_store_dwordx4).
template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[Vec<T>::N]) {
  T e[Vec<T>::N];
#pragma unroll
  for (int i = 0; i < Vec<T>::N; ++i) e[i] = from_f<T>(v[i]);
  u32x4 raw;
  __builtin_memcpy(&raw, e, 16);
  *reinterpret_cast<u32x4*>(p) = raw;
}

// The same store with the non-temporal hint: outputs written once and not read
// again by the kernel are streamed past the caches (global_store ... nt).
template <typename T>
__device__ __forceinline__ void store_vec_nt(T* p, const float (&v)[Vec<T>::N]) {
  T e[Vec<T>::N];
#pragma unroll
  for (int i = 0; i < Vec<T>::N; ++i) e[i] = from_f<T>(v[i]);
  u32x4 raw;
  __builtin_memcpy(&raw, e, 16);
  __builtin_nontemporal_store(raw, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ void store_raw_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

__device__ __forceinline__ u32x4 load_raw(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void store_raw(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// DPP row_ror:n moves lane (i + n) mod 16 of each 16-lane row into lane i.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over all 64 lanes of a wave; every lane gets the same value. The lanes
// of each 16-lane row are combined by a row_ror butterfly (8, 4, 2, 1), then
// the four row sums are read from lanes 0/16/32/48 in a fixed order, so the
// result is deterministic and uniform. Must be called with all lanes active.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f<0x128>(x);  // row_ror:8
  x += dpp_f<0x124>(x);  // row_ror:4
  x += dpp_f<0x122>(x);  // row_ror:2
  x += dpp_f<0x121>(x);  // row_ror:1
  const int xi = __builtin_bit_cast(int, x);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
  return (r0 + r1) + (r2 + r3);
}

// Sum over a workgroup of WAVES waves: wave_sum, one LDS slot per wave, then
// every thread adds the WAVES partials in a fixed order (deterministic). `part`
// must hold WAVES floats and must not be reused by a later call in the same
// kernel without a barrier; uniform control flow only.
template <int WAVES>
__device__ __forceinline__ float block_sum(float v, float* part) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int i = 0; i < WAVES; ++i) tot += part[i];
  return tot;
}

// Logistic sigmoid with the device library's accurate expf and an IEEE divide.
__device__ __forceinline__ float sigmoid_f(float t) { return 1.0f / (1.0f + expf(-t)); }

// Chain transcendentals: the device library's accurate functions, or the
// fastmath.h forms when the chain's output is fp16 (FAST).
template <bool FAST>
__device__ __forceinline__ float chain_exp(float v) { return FAST ? np_fast_exp(v) : expf(v); }
template <bool FAST>
__device__ __forceinline__ float chain_sigmoid(float v) {
  return FAST ? np_fast_sigmoid(v) : sigmoid_f(v);
}
template <bool FAST>
__device__ __forceinline__ float chain_tanh(float v) { return FAST ? np_fast_tanh(v) : tanhf(v); }

// Arithmetic of a RoPE rotation: fp32 for 16-bit data; fp64 for fp32 data,
// where an fp32 cos / sin (each within about one ulp) and two rounded products
// would put the rotated value u cos - w sin, when it cancels, further than
// 1e-6 relative from its exact value. In fp64 the result is rounded once to
// fp32. The angle itself stays the fp32 product fp32(pos) * inv_i.
template <typename T>
using rope_math_t = std::conditional_t<sizeof(T) == 4, double, float>;

__device__ inline void rope_sincos(float theta, float* s, float* c) { sincosf(theta, s, c); }
__device__ inline void rope_sincos(float theta, double* s, double* c) {
  sincos((double)theta, s, c);
}

}  // namespace np
