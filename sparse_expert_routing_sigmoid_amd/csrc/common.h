// Internal helpers of the MI355X MoE library: error reporting, bf16 and
// E4M3 conversions, wave-level reductions.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <cstdio>
#include <string>

#include "moe_mi355x.h"

namespace moe {

// ---------------------------------------------------------------- errors --
void set_error(const std::string& msg);
void clear_error();

#define MOE_REQUIRE(cond, code, msg)          \
  do {                                        \
    if (!(cond)) {                            \
      ::moe::set_error(std::string(__func__) + ": " + (msg)); \
      return (code);                          \
    }                                         \
  } while (0)

// SiLU(a) = a * sigmoid(a) of the expert FFNs, from the hardware base-2
// exponential and reciprocal (each within about 1 ulp): a few ulp in fp32,
// far below the bf16 / E4M3 rounding of h that follows.  Large negative a
// gives exp2 = inf, reciprocal 0 and SiLU = -0.
__device__ __forceinline__ float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}

// Data tensors (activations, weights, outputs, workspaces) are read and
// written with 16-byte vector accesses.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// A byte count that a 32-bit buffer offset can address.
inline bool fits31(unsigned long long bytes) { return bytes < (1ull << 31); }

// Checks the launch status after enqueueing kernels.
moe_status launch_status(const char* where);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// --------------------------------------------------------- conversions --
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (the gfx950 conversion instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two values in one v_cvt_pk_bf16_f32 (converting them one by one costs the
// conversion twice plus the masks and shifts that join the halves).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// E4M3FN (OCP): bias 7, 3 mantissa bits, largest finite 448, subnormal step 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  const uint32_t sign = (code & 0x80u) << 24;
  const uint32_t ef = (code >> 3) & 0xFu;
  const uint32_t mf = code & 0x7u;
  float mag;
  if (ef == 0) {
    mag = static_cast<float>(mf) * 0.001953125f;  // m * 2^-9, exact
  } else {
    mag = __uint_as_float(((ef + 120u) << 23) | (mf << 20));  // 2^(ef-7) * (1 + m/8)
  }
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// Values of magnitude <= 448 (x divided by its power-of-two scale, which is
// exact) to E4M3FN codes, round to nearest even, packed little-endian: the
// packed conversion of gfx950 (OCP E4M3).  Over every fp32 magnitude in
// [0, 448], both signs, it gives the same code as rounding the fp32 value to
// 3 mantissa bits with ties to even (subnormal step 2^-9 below 2^-6).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_cvt_pk_fp8_f32(c, d, __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false), true));
}

// Power-of-two tile scale: the smallest 2^k (k >= -126) with amax <= 448 * 2^k,
// or k = 0 for amax == 0.  With amax = 1.M * 2^(E-127): k = E - 135 when
// 1.M <= 1.75 (mantissa field <= 0x600000), else E - 134.  Returns k.
__host__ __device__ __forceinline__ int pow2_scale_exp(float amax) {
  uint32_t b;
  __builtin_memcpy(&b, &amax, 4);
  b &= 0x7FFFFFFFu;
  if (b == 0) return 0;
  const int E = (int)(b >> 23);
  if (E == 0) return -126;  // subnormal amax
  const int k = (b & 0x7FFFFFu) <= 0x600000u ? E - 135 : E - 134;
  return k < -126 ? -126 : k;
}

// 2^k as fp32 for -126 <= k <= 127.
__host__ __device__ __forceinline__ float exp2_int(int k) {
  const uint32_t b = (uint32_t)(k + 127) << 23;
  float f;
  __builtin_memcpy(&f, &b, 4);
  return f;
}

// ---------------------------------------------------------- wave helpers --
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    unsigned long long o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// Order-preserving map of a finite fp32 to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__host__ __device__ constexpr inline long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

}  // namespace moe
