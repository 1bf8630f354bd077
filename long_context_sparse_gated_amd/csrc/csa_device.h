// Device helpers shared by the kernels of libcsa (gfx950).
//
// Storage types: float (IEEE binary32) or bf16 carried as raw uint16 bits.
// Conversions round to nearest even.  Rotations (RoPE) of stored rows are
// computed in float64 from float64 cos/sin so that a stored bf16/float32
// value is the correctly rounded image of the exact rotation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa_internal.h"

namespace csa {

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float32 -> bf16, nearest even (the gfx950 conversion instruction).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

// two float32 -> packed bf16 pair (low half = a), nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// float64 -> float32 rounded to odd: the truncation toward zero with its last
// bit forced to 1 when inexact.  Rounding that value to any format with at
// least two fewer significand bits equals rounding the float64 directly.
__device__ __forceinline__ float f64_to_f32_odd(double d) {
  float f = (float)d;
  double back = (double)f;
  if (back != d) {
    uint32_t u = __float_as_uint(f);
    if (fabs(back) > fabs(d)) u -= 1u;  // step toward zero
    u |= 1u;
    f = __uint_as_float(u);
  }
  return f;
}

// float64 -> bf16 with a single rounding (nearest even).
__device__ __forceinline__ bf16_t f64_to_bf16(double d) {
  return f32_to_bf16(f64_to_f32_odd(d));
}

// Load / store one element of a storage type as float or double.
template <typename T> struct store_t;
template <> struct store_t<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
  static __device__ __forceinline__ void st64(float* p, double v) { *p = (float)v; }
  static __device__ __forceinline__ float cvt(float v) { return v; }
};
template <> struct store_t<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f32_to_bf16(v); }
  static __device__ __forceinline__ void st64(bf16_t* p, double v) { *p = f64_to_bf16(v); }
  static __device__ __forceinline__ float cvt(bf16_t v) { return bf16_to_f32(v); }
};

// Frequency of rope pair j of R rope channels, in float64: theta_j =
// base^(-2j/R), or with YaRN scaling by s = factor > 1,
// theta_j (1 - r_j) + (theta_j / s) r_j.  The ramp r_j rises linearly in j
// from 0 at lo to 1 at hi, lo and hi being the pair indices (rounded down and
// up, clamped to [0, R - 1]) at which a pair turns beta_fast and beta_slow
// times over the original context: c(n) = R ln(orig / (2 pi n)) / (2 ln base).
// Pairs below lo keep their frequency, pairs from hi on are slowed by s.
// [optimum-intel issue 1748, "What V4-Flash adds vs V3": YaRN, factor 16,
// 65k -> 1M context; the ramp is the YaRN method's]
__device__ __forceinline__ double rope_freq(const Rope& rp, int j, int R) {
  const double f = pow(rp.base, (-2.0 * (double)j) / (double)R);
  if (!(rp.factor > 1.0)) return f;
  double lo = floor((double)R * rp.ln_fast / rp.ln_base2);
  double hi = ceil((double)R * rp.ln_slow / rp.ln_base2);
  lo = lo > 0.0 ? lo : 0.0;
  hi = hi < (double)(R - 1) ? hi : (double)(R - 1);
  if (hi == lo) hi += 0.001;
  double r = ((double)j - lo) / (hi - lo);
  r = r < 0.0 ? 0.0 : (r > 1.0 ? 1.0 : r);
  return f * (1.0 - r) + (f / rp.factor) * r;
}

// (a, b) <- (a cos - b sin, a sin + b cos): multiplication by cos + i sin.
__device__ __forceinline__ void rot64(double& a, double& b, double c, double s) {
  double x = a * c - b * s;
  double y = a * s + b * c;
  a = x;
  b = y;
}

// Wave-wide reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace csa
