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

// round to nearest even (gfx950 converts in hardware: v_cvt_pk_bf16_f32)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_hw;
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_hw v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
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
// The angle p * f (f = theta^(-2i/R), fp64) is formed in revolutions and
// reduced to [0, 1) in fp64, so positions up to 2^20 keep the reduced angle
// exact to ~2^-35 of a turn; it is then rounded to fp32 and the hardware
// sine/cosine (which take revolutions) give (cos, sin).  Measured on gfx950
// over 2^20 positions x 32 frequencies: max abs error 2.6e-7 against fp64,
// the same as sincosf on the reduced angle (the fp32 rounding dominates).
__device__ __forceinline__ void rope_cs_f(double pos, double inv_freq, float sign, float *c, float *s) {
  const double inv_two_pi = 0.15915494309189533576888376337251;
  const double rev = pos * inv_freq * inv_two_pi;
  const float fr = (float)(rev - floor(rev));
  *c = __builtin_amdgcn_cosf(fr);
  *s = __builtin_amdgcn_sinf(fr) * sign;
}

// Inverse frequencies theta^(-2i/R) of the (at most 32) rope pairs, formed
// once on the host in fp64 and passed by value, so that every kernel that
// rotates uses the same table and none evaluates pow per element.
struct RopeTab {
  double f[32];
};
static inline RopeTab rope_table(double theta, int rope_dim) {
  RopeTab t;
  for (int i = 0; i < 32; ++i) t.f[i] = (i < rope_dim / 2) ? pow(theta, -2.0 * i / (double)rope_dim) : 0.0;
  return t;
}

// Rotate one interleaved rope pair by the angle whose (cos, sin) is (cs, sn).
// Written with explicit fmaf so that every kernel that rotates (the rope
// kernel, the compressor epilogue, the cache writer) rounds identically.
__device__ __forceinline__ void rope_rotate(float &x0, float &x1, float cs, float sn) {
  const float a = fmaf(x0, cs, -(x1 * sn)), b = fmaf(x0, sn, x1 * cs);
  x0 = a;
  x1 = b;
}

// One token of the compressor's per-channel online softmax: gate g (z + bias)
// and candidate c; the pooled value is acc / den once the window is done.
// Shared by the batch compressor and the streaming cache writer so that both
// produce the same bits for an entry.
struct PoolAcc {
  float mx, den, acc;
};
__device__ __forceinline__ PoolAcc pool_init() { return PoolAcc{-INFINITY, 0.f, 0.f}; }
__device__ __forceinline__ void pool_step(PoolAcc &a, float g, float c) {
  if (g > a.mx) {
    const float r = __expf(a.mx - g);
    a.den *= r;
    a.acc *= r;
    a.mx = g;
  }
  const float e = __expf(g - a.mx);
  a.den += e;
  a.acc = fmaf(e, c, a.acc);
}

// ---- storage encoders (quantise-on-write) ----
// E4M3 code of v, round to nearest even, saturating at 448 (the code 0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
  const uint32_t sgn = (__float_as_uint(v) >> 31) << 7;
  const float a = fabsf(v);
  if (!(a < 464.f)) return sgn | 0x7Eu;          // at or past the 448 | NaN midpoint: 448
  if (a < 0.015625f) return sgn | (uint32_t)rintf(a * 512.f);   // subnormal steps of 2^-9 (8 = 2^-6)
  int ex = (int)(__float_as_uint(a) >> 23) - 127;              // floor(log2 a), a normal
  const float q = rintf((ldexpf(a, -ex) - 1.f) * 8.f);          // 3 mantissa bits, ties to even
  int mq = (int)q;
  if (mq == 8) {
    mq = 0;
    ++ex;
  }
  if (ex > 8 || (ex == 8 && mq == 7)) return sgn | 0x7Eu;
  return sgn | ((uint32_t)(ex + 7) << 3) | (uint32_t)mq;
}

// E2M1 code of v for a block scale 2^e (nearest, ties to even, saturating at
// 6, no negative zero).
__device__ __forceinline__ uint32_t e2m1_encode(float v, int e) {
  const float a = fabsf(ldexpf(v, -e));
  // thresholds between grid points 0 .5 1 1.5 2 3 4 6; '>' at a midpoint below
  // an odd code, '>=' below an even one
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) + (uint32_t)(a >= 1.75f) +
                     (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
  return c ? (c | ((__float_as_uint(v) >> 31) << 3)) : 0u;
}

// FP8R row scale from the row's largest |x| over the E4M3 channels.
__device__ __forceinline__ float fp8r_scale(float amax) { return amax > 0.f ? amax / 448.f : 1.f; }

// MXFP4 block exponent from the block's largest |x|: floor(log2 amax) - 2,
// clamped to the E8M0 range (-127 for an all-zero block).
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int k2;
  frexpf(amax, &k2);   // amax = f 2^k2, f in [0.5, 1)
  return min(127, max(-127, k2 - 3));
}

__device__ __forceinline__ int64_t row_bytes(int dtype, int dim, int tail) {
  switch (dtype) {
  case DSV4_F32: return 4LL * dim;
  case DSV4_BF16: return 2LL * dim;
  case DSV4_F16: return 2LL * dim;
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

// max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48):
// two row-swapping permutes on the VALU instead of two LDS round trips
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// max(x, 0) by the bit pattern: non-negative floats order like their bit
// patterns read as signed integers and negative ones read as negative, so one
// integer maximum gives the result without the NaN canonicalisation a float
// maximum of a matrix-core result needs (inputs here are finite)
__device__ __forceinline__ float relu_f(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

}  // namespace dsv4

// Host-side helpers shared by the launchers (defined in dsv4_api.cpp)
namespace dsv4host {
int fail(int code, const char *fmt, ...);
int check_launch(const char *what);
}  // namespace dsv4host
