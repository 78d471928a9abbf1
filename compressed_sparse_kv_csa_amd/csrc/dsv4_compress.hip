// dsv4_compress.hip -- KV compressor (softmax-gated pooling with a learned
// position bias) and the partial interleaved RoPE kernel, for gfx950.
//
// HF DeepSeek-V4 page, "Hybrid attention": CSA pools every m = 4 tokens over
// overlapping windows, HCA every m' = 128 tokens over non-overlapping windows;
// insight.ai.kr: the pooling is softmax-gated with a learned per-position bias.
//
// Design: HBM-bound streaming.  One thread owns one (entry, channel pair) and
// walks the entry's window with an online softmax (running max, rescaled sum),
// so every c/z element is read once per window it belongs to (twice for the
// overlapping CSA windows, the second read coming from L2).  Consecutive
// threads own consecutive channel pairs: each window step is one coalesced
// 4-byte (bf16x2) or 8-byte (f32x2) load per thread.  The rope epilogue
// rotates the pair at P_s = pos0 + s*m with an fp64 angle.
#include "dsv4_common.h"

namespace dsv4 {

template <typename T>
struct Pair;
template <>
struct Pair<float> {
  static __device__ __forceinline__ float2 load(const void *p, int64_t i) {
    return reinterpret_cast<const float2 *>(p)[i];
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, float a, float b) {
    reinterpret_cast<float2 *>(p)[i] = make_float2(a, b);
  }
};
struct F16T {};   // tag: IEEE half storage
template <>
struct Pair<F16T> {
  static __device__ __forceinline__ float2 load(const void *p, int64_t i) {
    const uint32_t u = reinterpret_cast<const uint32_t *>(p)[i];
    _Float16 a, b;
    const uint16_t lo = (uint16_t)(u & 0xFFFF), hi = (uint16_t)(u >> 16);
    __builtin_memcpy(&a, &lo, 2);
    __builtin_memcpy(&b, &hi, 2);
    return make_float2((float)a, (float)b);
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, float a, float b) {
    reinterpret_cast<uint32_t *>(p)[i] = pack_f16x2(a, b);
  }
};
template <>
struct Pair<uint16_t> {
  static __device__ __forceinline__ float2 load(const void *p, int64_t i) {
    uint32_t u = reinterpret_cast<const uint32_t *>(p)[i];
    return make_float2(bf16_to_f32((uint16_t)(u & 0xFFFF)), bf16_to_f32((uint16_t)(u >> 16)));
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, float a, float b) {
    reinterpret_cast<uint32_t *>(p)[i] = pack_bf16x2(a, b);
  }
};

// grid: x = entry * pair_blocks + pair block, y = sequence
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void k_compress(const void *__restrict__ c, const void *__restrict__ z,
                                                  const float *__restrict__ bias, int S, int dim, int m,
                                                  int overlap, int rope_dim, RopeTab tab,
                                                  const int64_t *__restrict__ pos0, void *__restrict__ pool) {
  const int half = dim >> 1;
  const int pblocks = (half + blockDim.x - 1) / blockDim.x;
  const int s = blockIdx.x / pblocks, b = blockIdx.y;
  const int pr = (blockIdx.x % pblocks) * blockDim.x + threadIdx.x;   // channel pair
  if (pr >= half) return;
  const int N = S / m;
  const int t0 = overlap ? (s - 1) * m : s * m;
  const int width = overlap ? 2 * m : m;
  const int jlo = t0 < 0 ? -t0 : 0;
  const int64_t rowbase = (int64_t)b * S;
  PoolAcc a0 = pool_init(), a1 = pool_init();
  // window tokens in batches of 8: a batch's loads are all issued before its
  // online-softmax steps, which run in token order as one at a time would
  // (batches of 16 were measured slower: 38 -> 54 us at S = 65536)
  const int jhi = width < S - t0 ? width : S - t0;   // tokens t0 + j < S
  int j = jlo;
  for (; j + 8 <= jhi; j += 8) {
    float2 zz[8], cc[8], bb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t e = (rowbase + t0 + j + u) * half + pr;
      zz[u] = Pair<TI>::load(z, e);
      cc[u] = Pair<TI>::load(c, e);
      bb[u] = reinterpret_cast<const float2 *>(bias)[(int64_t)(j + u) * half + pr];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      pool_step(a0, zz[u].x + bb[u].x, cc[u].x);
      pool_step(a1, zz[u].y + bb[u].y, cc[u].y);
    }
  }
  for (; j < jhi; ++j) {
    const int64_t e = (rowbase + t0 + j) * half + pr;
    const float2 zz = Pair<TI>::load(z, e);
    const float2 cc = Pair<TI>::load(c, e);
    const float2 bb = reinterpret_cast<const float2 *>(bias)[(int64_t)j * half + pr];
    pool_step(a0, zz.x + bb.x, cc.x);
    pool_step(a1, zz.y + bb.y, cc.y);
  }
  float o0 = a0.acc / a0.den, o1 = a1.acc / a1.den;
  const int d0 = 2 * pr;
  if (rope_dim > 0 && d0 >= dim - rope_dim) {
    const int pair = (d0 - (dim - rope_dim)) >> 1;
    const double P = (double)((pos0 ? pos0[b] : 0) + (int64_t)s * m);
    float cs, sn;
    rope_cs_f(P, tab.f[pair], 1.f, &cs, &sn);
    rope_rotate(o0, o1, cs, sn);
  }
  Pair<TO>::store(pool, ((int64_t)b * N + s) * half + pr, o0, o1);
}

// grid: x = pair blocks, y = row blocks.  y may alias x.
template <typename T, typename TO>
__global__ __launch_bounds__(256) void k_rope(const void *x, void *y, int64_t n_rows,
                                              int dim, int rope_dim, const int64_t *__restrict__ pos,
                                              RopeTab tab, float sign) {
  const int half = dim >> 1;
  const int pr = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t r = blockIdx.y;
  if (pr >= half || r >= n_rows) return;
  const int64_t e = r * half + pr;
  float2 v = Pair<T>::load(x, e);
  const int d0 = 2 * pr;
  if (d0 >= dim - rope_dim) {
    float cs, sn;
    rope_cs_f((double)pos[r], tab.f[(d0 - (dim - rope_dim)) >> 1], sign, &cs, &sn);
    rope_rotate(v.x, v.y, cs, sn);
  }
  Pair<TO>::store(y, e, v.x, v.y);
}

// Eight channels (16-byte bf16/fp16 or 2 x 16-byte fp32 accesses) per thread,
// rows flattened into one grid dimension: for dim % 8 == 0 and 16-byte
// aligned rows.  Same arithmetic per pair as k_rope.
template <typename T>
struct Vec8;
template <>
struct Vec8<uint16_t> {   // bf16
  static __device__ __forceinline__ void load(const void *p, int64_t i, float (&v)[8]) {
    const u32x4 u = reinterpret_cast<const u32x4 *>(p)[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_to_f32((uint16_t)(w[k] & 0xFFFF));
      v[2 * k + 1] = bf16_to_f32((uint16_t)(w[k] >> 16));
    }
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, const float (&v)[8]) {
    reinterpret_cast<u32x4 *>(p)[i] =
        u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
  }
};
template <>
struct Vec8<F16T> {
  static __device__ __forceinline__ void load(const void *p, int64_t i, float (&v)[8]) {
    const u32x4 u = reinterpret_cast<const u32x4 *>(p)[i];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      _Float16 a, b;
      const uint16_t lo = (uint16_t)(w[k] & 0xFFFF), hi = (uint16_t)(w[k] >> 16);
      __builtin_memcpy(&a, &lo, 2);
      __builtin_memcpy(&b, &hi, 2);
      v[2 * k] = (float)a;
      v[2 * k + 1] = (float)b;
    }
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, const float (&v)[8]) {
    reinterpret_cast<u32x4 *>(p)[i] =
        u32x4{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3]), pack_f16x2(v[4], v[5]), pack_f16x2(v[6], v[7])};
  }
};
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const void *p, int64_t i, float (&v)[8]) {
    const f32x4 a = reinterpret_cast<const f32x4 *>(p)[2 * i], b = reinterpret_cast<const f32x4 *>(p)[2 * i + 1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
  }
  static __device__ __forceinline__ void store(void *p, int64_t i, const float (&v)[8]) {
    reinterpret_cast<f32x4 *>(p)[2 * i] = f32x4{v[0], v[1], v[2], v[3]};
    reinterpret_cast<f32x4 *>(p)[2 * i + 1] = f32x4{v[4], v[5], v[6], v[7]};
  }
};
// With 512 channels a wave covers exactly one row (64 lanes x 8 channels):
// the row's rope angles are then evaluated once per pair, lane i taking pair
// i, and handed to the lanes that rotate through cross-lane reads, instead of
// eight lanes evaluating four angles each while the rest of the wave waits.
template <typename T, typename TO>
__global__ __launch_bounds__(256) void k_rope8(const void *x, void *y, int64_t n_rows, int dim, int rope_dim,
                                               const int64_t *__restrict__ pos, RopeTab tab, float sign) {
  const int per = dim >> 3;   // 8-channel groups per row
  const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (it >= n_rows * per) return;   // with per == 64, whole waves
  if (per == 64) {
    const int64_t r = it >> 6;
    const int lane = (int)threadIdx.x & 63, d0 = 8 * lane, lo = dim - rope_dim;
    float v[8];
    Vec8<T>::load(x, it, v);
    float cs = 1.f, sn = 0.f;
    if (lane < (rope_dim >> 1)) rope_cs_f((double)pos[r], tab.f[lane], sign, &cs, &sn);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = d0 + 2 * k, pr = d >= lo ? (d - lo) >> 1 : 0;
      const float c_k = __shfl(cs, pr, 64), s_k = __shfl(sn, pr, 64);   // every lane takes part
      if (d >= lo) rope_rotate(v[2 * k], v[2 * k + 1], c_k, s_k);
    }
    Vec8<TO>::store(y, it, v);
    return;
  }
  const int64_t r = it / per;
  const int d0 = 8 * (int)(it - r * per);
  float v[8];
  Vec8<T>::load(x, it, v);
  if (d0 + 8 > dim - rope_dim) {
    const double p = (double)pos[r];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int d = d0 + 2 * k;
      if (d >= dim - rope_dim) {
        float cs, sn;
        rope_cs_f(p, tab.f[(d - (dim - rope_dim)) >> 1], sign, &cs, &sn);
        rope_rotate(v[2 * k], v[2 * k + 1], cs, sn);
      }
    }
  }
  Vec8<TO>::store(y, it, v);
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

int launch_compress(const void *c, const void *z, int in_dtype, const float *bias, int B, int S, int dim,
                    int m, int overlap, int rope_dim, double theta, const int64_t *pos0, void *pool,
                    int out_dtype, hipStream_t st) {
  const int N = S / m;
  if (B == 0 || N == 0) return DSV4_OK;
  dim3 grid((unsigned)(N * ((dim / 2 + 255) / 256)), B), block(256);
  const RopeTab tab = rope_table(theta, rope_dim);
#define DSV4_CMP(TI, TO)                                                                               \
  hipLaunchKernelGGL((k_compress<TI, TO>), grid, block, 0, st, c, z, bias, S, dim, m, overlap, rope_dim, \
                     tab, pos0, pool)
  if (in_dtype == DSV4_F32) {
    if (out_dtype == DSV4_F32) DSV4_CMP(float, float);
    else if (out_dtype == DSV4_BF16) DSV4_CMP(float, uint16_t);
    else DSV4_CMP(float, F16T);
  } else {
    if (out_dtype == DSV4_F32) DSV4_CMP(uint16_t, float);
    else if (out_dtype == DSV4_BF16) DSV4_CMP(uint16_t, uint16_t);
    else DSV4_CMP(uint16_t, F16T);
  }
#undef DSV4_CMP
  return check_launch("k_compress");
}

int launch_rope(const void *x, int x_dtype, void *y, int y_dtype, int64_t n_rows, int dim, int rope_dim,
                const int64_t *pos, double theta, int inverse, hipStream_t st) {
  if (n_rows == 0) return DSV4_OK;
  const float sign = inverse ? -1.f : 1.f;
  const RopeTab tab = rope_table(theta, rope_dim);
  if (dim % 8 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)y & 15) == 0) {
    const int64_t items = n_rows * (dim / 8);
    dim3 grid((unsigned)((items + 255) / 256)), block(256);
#define DSV4_ROPE8(TI, TO) hipLaunchKernelGGL((k_rope8<TI, TO>), grid, block, 0, st, x, y, n_rows, dim, rope_dim, pos, tab, sign)
    if (x_dtype == DSV4_F32) {
      if (y_dtype == DSV4_F32) DSV4_ROPE8(float, float);
      else if (y_dtype == DSV4_BF16) DSV4_ROPE8(float, uint16_t);
      else DSV4_ROPE8(float, F16T);
    } else {
      if (y_dtype == DSV4_F32) DSV4_ROPE8(uint16_t, float);
      else if (y_dtype == DSV4_BF16) DSV4_ROPE8(uint16_t, uint16_t);
      else DSV4_ROPE8(uint16_t, F16T);
    }
#undef DSV4_ROPE8
    return check_launch("k_rope8");
  }
  int64_t done = 0;
  while (done < n_rows) {   // grid.y is limited to 65535 rows per launch
    const int64_t n = (n_rows - done) < 65535 ? (n_rows - done) : 65535;
    dim3 grid((dim / 2 + 255) / 256, (unsigned)n), block(256);
    const void *xs = (const char *)x + done * (int64_t)dim * (x_dtype == DSV4_F32 ? 4 : 2);
    void *ys = (char *)y + done * (int64_t)dim * (y_dtype == DSV4_F32 ? 4 : 2);
#define DSV4_ROPE(TI, TO) \
  hipLaunchKernelGGL((k_rope<TI, TO>), grid, block, 0, st, xs, ys, n, dim, rope_dim, pos + done, tab, sign)
    if (x_dtype == DSV4_F32) {
      if (y_dtype == DSV4_F32) DSV4_ROPE(float, float);
      else if (y_dtype == DSV4_BF16) DSV4_ROPE(float, uint16_t);
      else DSV4_ROPE(float, F16T);
    } else {
      if (y_dtype == DSV4_F32) DSV4_ROPE(uint16_t, float);
      else if (y_dtype == DSV4_BF16) DSV4_ROPE(uint16_t, uint16_t);
      else DSV4_ROPE(uint16_t, F16T);
    }
#undef DSV4_ROPE
    done += n;
  }
  return check_launch("k_rope");
}

}  // namespace dsv4host
