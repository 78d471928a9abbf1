// dsv4_common.h -- device helpers shared by the gfx950 kernels of libdsv4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsv4.h"

namespace dsv4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr float kLog2e = 1.4426950408889634f;

// ---- bfloat16 <-> float (bit patterns kept in uint16_t) ----
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// round to nearest even; inputs are finite
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// two floats -> packed IEEE fp16 pair (round to nearest even)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = (_Float16)lo, b = (_Float16)hi;
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// ---- OCP FP8 E4M3 (fn) -> float, exact for every finite code ----
// normal: (-1)^s 2^(e-7) (1 + m/8); subnormal (e = 0): (-1)^s m 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) {
  uint32_t s = (v & 0x80u) << 24;
  uint32_t e = (v >> 3) & 15u, m = v & 7u;
  float mag = (e == 0) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | s);
}

// ---- rope angle -> (cos, sin) in fp32 ----
// The angle p * f (f = theta^(-2i/R), fp64) is formed and reduced modulo 2 pi in
// fp64, so positions up to 2^20 keep an angle error below a microradian; the
// reduced angle is then rounded to fp32 (< 4e-7 rad) for sin/cos.
__device__ __forceinline__ void rope_cs_f(double pos, double inv_freq, float sign, float *c, float *s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = pos * inv_freq;
  a = a - two_pi * floor(a / two_pi);
  float sn, cs;
  sincosf((float)a, &sn, &cs);
  *c = cs;
  *s = sn * sign;
}

__device__ __forceinline__ void rope_cs(double pos, int pair, int rope_dim, double theta, float sign,
                                        float *c, float *s) {
  rope_cs_f(pos, pow(theta, -2.0 * (double)pair / (double)rope_dim), sign, c, s);
}

__device__ __forceinline__ int64_t row_bytes(int dtype, int dim, int tail) {
  switch (dtype) {
  case DSV4_F32: return 4LL * dim;
  case DSV4_BF16: return 2LL * dim;
  case DSV4_FP8R: return (int64_t)(dim - tail) + 2LL * tail;
  case DSV4_MXFP4: return dim / 2;
  }
  return 0;
}

// Warp (wavefront of 64) reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace dsv4

// Host-side helpers shared by the launchers (defined in dsv4_api.cpp)
namespace dsv4host {
int fail(int code, const char *fmt, ...);
int check_launch(const char *what);
}  // namespace dsv4host
