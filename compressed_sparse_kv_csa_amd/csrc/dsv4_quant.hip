// dsv4_quant.hip -- quantise-on-write of stored rows for gfx950.
//
// insight.ai.kr deep dive: the KV cache is FP8 with the RoPE channels kept in
// BF16; MarkTechPost: the Lightning Indexer's query/key path is MXFP4.  The
// pages give the formats, not the scale recipe; the readings used:
//   FP8R : one fp32 scale per row, s = amax/448 over the E4M3 channels (1 for
//          an all-zero row); each code is the E4M3 value nearest to x/s, ties
//          to the even code, sign of x/s kept, saturated at 448; the trailing
//          `tail` channels are stored as bf16 (round to nearest even).
//   MXFP4: blocks of 32 channels share the OCP MX scale 2^(floor(log2 amax)-2)
//          (2^-127 for an all-zero block, exponent clamped to [-127, 127]);
//          each code is the E2M1 value nearest to x/scale, saturated at 6,
//          ties to the even code, no negative zero; low nibble = even channel.
//
// k_quantize: one wave per row, lane l holds channels [E*l, E*l + E) with
// E = dim/64, so an MX block of 32 channels is 32/E consecutive lanes and the
// row and block maxima are cross-lane reductions.
#include "dsv4_common.h"

namespace dsv4 {

template <int XD>
__device__ __forceinline__ float load_x(const void *x, int64_t i) {
  if constexpr (XD == DSV4_F32) return reinterpret_cast<const float *>(x)[i];
  if constexpr (XD == DSV4_BF16) return bf16_to_f32(reinterpret_cast<const uint16_t *>(x)[i]);
  return (float)reinterpret_cast<const _Float16 *>(x)[i];
}

// grid ceil(n/4), block 256: wave w of block b quantises row 4b + w.
template <int XD, bool MX>
__global__ __launch_bounds__(256) void k_quantize(const void *x, int64_t n, int dim, int tail, uint8_t *rows,
                                                  float *row_scale, uint8_t *blk_scale) {
  constexpr int EMAX = 8;   // dim <= 512
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= n) return;
  const int E = dim / 64;
  float v[EMAX];
#pragma unroll
  for (int k = 0; k < EMAX; ++k) v[k] = k < E ? load_x<XD>(x, r * dim + E * lane + k) : 0.f;
  if constexpr (!MX) {
    const int nq = dim - tail;   // E4M3 channels
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < EMAX; ++k)
      if (k < E && E * lane + k < nq) am = fmaxf(am, fabsf(v[k]));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const float s = fp8r_scale(am);
    if (lane == 0) row_scale[r] = s;
    uint8_t *o = rows + r * (int64_t)(nq + 2 * tail);
#pragma unroll
    for (int k = 0; k < EMAX; ++k) {
      if (k >= E) break;
      const int d = E * lane + k;
      if (d < nq) {
        o[d] = (uint8_t)e4m3_encode(v[k] / s);
      } else {
        const uint16_t h = f32_to_bf16(v[k]);
        o[nq + 2 * (d - nq)] = (uint8_t)(h & 0xFF);
        o[nq + 2 * (d - nq) + 1] = (uint8_t)(h >> 8);
      }
    }
  } else {
    // block max over the 32/E lanes of each 32-channel block
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < EMAX; ++k)
      if (k < E) am = fmaxf(am, fabsf(v[k]));
    for (int o = 1; o < 32 / E; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const int e = mx_exponent(am);
    if ((E * lane) % 32 == 0) blk_scale[r * (dim / 32) + (E * lane) / 32] = (uint8_t)(e + 127);
    uint8_t *o = rows + r * (int64_t)(dim / 2);
    if (E == 1) {   // a lane holds one channel: pair it with its odd neighbour
      const uint32_t c = e2m1_encode(v[0], e);
      const uint32_t hi = (uint32_t)__shfl_down((int)c, 1, 64);
      if ((lane & 1) == 0) o[lane / 2] = (uint8_t)(c | (hi << 4));
    } else {
#pragma unroll
      for (int k = 0; k < EMAX; k += 2) {
        if (k >= E) break;
        const int d = E * lane + k;
        o[d / 2] = (uint8_t)(e2m1_encode(v[k], e) | (e2m1_encode(v[k + 1], e) << 4));
      }
    }
  }
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

int launch_quantize(const void *x, int x_dtype, int64_t n, int dim, int tail, void *rows, float *row_scale,
                    uint8_t *blk_scale, int out_dtype, hipStream_t st) {
  if (n == 0) return DSV4_OK;
  const bool mx = out_dtype == DSV4_MXFP4;
  dim3 grid((unsigned)((n + 3) / 4)), block(256);
  uint8_t *o = (uint8_t *)rows;
#define DSV4_Q(XD)                                                                                         \
  if (mx) hipLaunchKernelGGL((k_quantize<XD, true>), grid, block, 0, st, x, n, dim, tail, o, row_scale, blk_scale); \
  else hipLaunchKernelGGL((k_quantize<XD, false>), grid, block, 0, st, x, n, dim, tail, o, row_scale, blk_scale);
  switch (x_dtype) {
  case DSV4_F32: DSV4_Q(DSV4_F32) break;
  case DSV4_BF16: DSV4_Q(DSV4_BF16) break;
  default: DSV4_Q(DSV4_F16) break;
  }
#undef DSV4_Q
  return check_launch("k_quantize");
}

}  // namespace dsv4host
