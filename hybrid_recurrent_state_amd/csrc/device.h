// Device helpers shared by the HIP translation units (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace hrs {

// Error of the launch just issued on this thread; recorded for
// hrs_last_hip_error().
inline hipError_t launch_error() {
  const hipError_t e = hipGetLastError();
  set_last_hip_error(static_cast<int>(e));
  return e;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 -> f32 is exact: the bf16 pattern is the upper half of the f32.
// Makes the compiler read the given kernel-argument values here, as one batch
// of scalar loads, instead of after the kernel's first branch (an early-exit
// test loads its bound first and the pointers only behind it): every later
// batch of argument loads is one more dependent memory round trip before the
// first data load of the launch.
template <typename T>
__device__ __forceinline__ void arg_in_register(const T& v) {
  asm volatile("" : : "s"(v));
}
template <typename... Ts>
__device__ __forceinline__ void args_in_registers(const Ts&... v) {
  (arg_in_register(v), ...);
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_one(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }

// Load one element of a float or bf16 array as f32.
template <typename T> __device__ __forceinline__ float load_elem(const T* p, size_t i);
template <> __device__ __forceinline__ float load_elem<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
  return bf16_one(p[i]);
}

// Eight consecutive elements as f32 (16 B of bf16 or 2 x 16 B of f32);
// the source must be 16-byte aligned.
template <typename T> __device__ __forceinline__ void load8(const T* p, float* o);
template <> __device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* o) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
  o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x);
  o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
  o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z);
  o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float* o) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
  const f32x4 y = *reinterpret_cast<const f32x4*>(p + 4);
  o[0] = x.x; o[1] = x.y; o[2] = x.z; o[3] = x.w;
  o[4] = y.x; o[5] = y.y; o[6] = y.z; o[7] = y.w;
}

// SiLU z / (1 + e^-z) from the hardware base-2 exponential and reciprocal:
// e^-z = 2^(-z log2 e); a few ulp from the correctly rounded value (large
// negative z gives -0 through 1 / inf, large positive z gives z). The conv
// kernels and the fused layer's staging share it, so every launch shape and
// path gives a request the same values.
__device__ __forceinline__ float silu_fast(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Cross-lane move inside a 16-lane DPP row. CTRL is a DPP control code:
// 0xB1 quad_perm[1,0,3,2], 0x4E quad_perm[2,3,0,1], 0x141 row_half_mirror,
// 0x140 row_mirror. Every lane has a valid source for these patterns.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Butterfly sum over aligned groups of N lanes (N in {4, 8, 16}). Every lane
// of a group ends with the same bits (IEEE addition is commutative), and the
// association order is fixed, so results are reproducible.
template <int N> __device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  x += dpp_mov<0xB1>(x);
  x += dpp_mov<0x4E>(x);
  if (N >= 8) x += dpp_mov<0x141>(x);
  if (N >= 16) x += dpp_mov<0x140>(x);
  return x;
}

}  // namespace hrs
