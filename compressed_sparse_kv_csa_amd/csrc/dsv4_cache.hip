// dsv4_cache.hip -- streaming maintenance of the decode caches for gfx950.
//
// HF DeepSeek-V4 page, "Cache layers": a compressed-attention layer carries a
// sliding window of K=V rows and, per compressed stream, a buffer of the newest
// tokens, the pool and its count (with overlap state for CSA) from one forward
// call to the next.  insight.ai.kr deep dive: the stored KV is FP8 with BF16
// rope channels; MarkTechPost summary: MXFP4 indexer keys.
//
// One append = two launches on the caller's stream:
//   k_cache_write : one workgroup per work item of a sequence -- a window
//                   token to rotate and quantise into its ring slot, or a
//                   compressed entry whose window closes in this append, pooled
//                   from the buffered older tokens and the new inputs, rotated
//                   and quantised into the pool.  Thread p owns channel pair p.
//   k_cache_state : one workgroup per sequence -- copies the newest span
//                   tokens into the buffers (after every reader of the old
//                   buffer has finished: stream order) and advances len, the
//                   pool counts and the window count / first token.
// The entry arithmetic is the batch compressor's (pool_step, rope_rotate) and
// the encoders are the quantiser's, so a streamed cache equals
// dsv4_compress + dsv4_quantize (and dsv4_rope + dsv4_quantize for the window)
// bit for bit.
#include "dsv4_common.h"

namespace dsv4 {

struct CacheStreamD {
  int dim, rope, dtype, tail;
  RopeTab tab;   // inverse frequencies of this stream's rope pairs
  const float *bias;
  float *buf;
  uint8_t *pool;
  float *rsc;
  uint8_t *bsc;
  int64_t cap;
  int32_t *count;
  const void *c, *z;   // inputs [B, n, dim]
};

struct CacheArgs {
  int B, n, m, overlap, span;
  double theta;
  const int64_t *pos0;
  int32_t *len;
  const int32_t *n_new;
  // window ring
  const void *kv;
  uint8_t *win;
  float *wsc;
  int wdtype, wtail, wcap, wdim, wrope;
  RopeTab wtab;
  int32_t *wcount, *wfirst;
  // work items per sequence: [0, nwi) window tokens, then nei entries per stream
  int nwi, nei, ns;
  CacheStreamD st[2];
};

template <bool BF>
__device__ __forceinline__ float2 load_pair(const void *p, int64_t pair_index) {
  if constexpr (BF) {
    const uint32_t u = reinterpret_cast<const uint32_t *>(p)[pair_index];
    return make_float2(bf16_to_f32((uint16_t)(u & 0xFFFF)), bf16_to_f32((uint16_t)(u >> 16)));
  } else {
    return reinterpret_cast<const float2 *>(p)[pair_index];
  }
}

// Store one row held one channel pair per thread (pair p = threadIdx.x, active
// when p < dim/2) in `dtype`.  Block-uniform control flow: FP8R takes the row
// maximum across the workgroup.  `red` is 4 floats of LDS.
__device__ __forceinline__ void store_row_pairs(int dtype, int dim, int tail, uint8_t *row, float *rsc,
                                                uint8_t *bsc, float v0, float v1, bool active, float *red) {
  const int p = threadIdx.x, d0 = 2 * p;
  switch (dtype) {
  case DSV4_F32:
    if (active) reinterpret_cast<float2 *>(row)[p] = make_float2(v0, v1);
    return;
  case DSV4_BF16:
    if (active) reinterpret_cast<uint32_t *>(row)[p] = pack_bf16x2(v0, v1);
    return;
  case DSV4_F16:
    if (active) reinterpret_cast<uint32_t *>(row)[p] = pack_f16x2(v0, v1);
    return;
  case DSV4_FP8R: {
    const int nq = dim - tail;   // even: a pair is all E4M3 or all bf16
    float am = (active && d0 < nq) ? fmaxf(fabsf(v0), fabsf(v1)) : 0.f;
    am = wave_max(am);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = am;
    __syncthreads();
    am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = fp8r_scale(am);
    if (threadIdx.x == 0) *rsc = s;
    if (active) {
      if (d0 < nq) {
        const uint32_t c = e4m3_encode(v0 / s) | (e4m3_encode(v1 / s) << 8);
        *reinterpret_cast<uint16_t *>(row + d0) = (uint16_t)c;
      } else {
        *reinterpret_cast<uint32_t *>(row + nq + 2 * (d0 - nq)) = pack_bf16x2(v0, v1);
      }
    }
    return;
  }
  case DSV4_MXFP4: {
    // a 32-channel block is 16 consecutive threads
    float am = active ? fmaxf(fabsf(v0), fabsf(v1)) : 0.f;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    const int e = mx_exponent(am);
    if (active) {
      if ((d0 & 31) == 0) bsc[d0 / 32] = (uint8_t)(e + 127);
      row[p] = (uint8_t)(e2m1_encode(v0, e) | (e2m1_encode(v1, e) << 4));
    }
    return;
  }
  }
}

// grid (nwi + ns*nei, B), block 256
template <bool BF>
__global__ __launch_bounds__(256) void k_cache_write(CacheArgs A) {
  __shared__ float red[4];
  const int b = blockIdx.y, item = blockIdx.x, p = threadIdx.x;
  const int L = A.len[b];
  const int nb = A.n_new ? min(A.n_new[b], A.n) : A.n;
  if (nb <= 0) return;
  const int64_t pos0 = A.pos0 ? A.pos0[b] : 0;
  if (item < A.nwi) {
    // window token: the newest min(nb, wcap) tokens of this append
    const int nw = min(nb, A.wcap);
    if (item >= nw) return;
    const int i = nb - nw + item, j = L + i;
    const int half = A.wdim >> 1, d0 = 2 * p;
    const bool active = p < half;
    float2 v = make_float2(0.f, 0.f);
    if (active) {
      v = load_pair<BF>(A.kv, ((int64_t)b * A.n + i) * half + p);
      if (A.wrope > 0 && d0 >= A.wdim - A.wrope) {
        float cs, sn;
        rope_cs_f((double)(pos0 + j), A.wtab.f[(d0 - (A.wdim - A.wrope)) >> 1], 1.f, &cs, &sn);
        rope_rotate(v.x, v.y, cs, sn);
      }
    }
    const int64_t slot = (int64_t)b * A.wcap + (j % A.wcap);
    store_row_pairs(A.wdtype, A.wdim, A.wtail, A.win + slot * row_bytes(A.wdtype, A.wdim, A.wtail),
                    A.wsc ? A.wsc + slot : nullptr, nullptr, v.x, v.y, active, red);
    return;
  }
  const int si = (item - A.nwi) / A.nei, e = (item - A.nwi) % A.nei;
  if (si >= A.ns) return;
  const CacheStreamD &S = A.st[si];
  const int m = A.m;
  const int s = L / m + e;
  if ((int64_t)(s + 1) * m > (int64_t)L + nb || s >= S.cap) return;   // not closed in this append, or no room
  const int half = S.dim >> 1, d0 = 2 * p;
  const bool active = p < half;
  const int t0 = A.overlap ? (s - 1) * m : s * m;
  const int width = A.overlap ? 2 * m : m;
  const int jlo = t0 < 0 ? -t0 : 0;
  float o0 = 0.f, o1 = 0.f;
  if (active) {
    PoolAcc a0 = pool_init(), a1 = pool_init();
    for (int jj = jlo; jj < width; ++jj) {
      const int t = t0 + jj;
      float2 zz, cc;
      if (t >= L) {   // a token of this append
        const int64_t pi = ((int64_t)b * A.n + (t - L)) * half + p;
        zz = load_pair<BF>(S.z, pi);
        cc = load_pair<BF>(S.c, pi);
      } else {        // a buffered token
        const float *br = S.buf + (((int64_t)b * A.span + (t % A.span)) * 2) * S.dim;
        cc = reinterpret_cast<const float2 *>(br)[p];
        zz = reinterpret_cast<const float2 *>(br + S.dim)[p];
      }
      const float2 bb = reinterpret_cast<const float2 *>(S.bias)[(int64_t)jj * half + p];
      pool_step(a0, zz.x + bb.x, cc.x);
      pool_step(a1, zz.y + bb.y, cc.y);
    }
    o0 = a0.acc / a0.den;
    o1 = a1.acc / a1.den;
    if (S.rope > 0 && d0 >= S.dim - S.rope) {
      float cs, sn;
      rope_cs_f((double)(pos0 + (int64_t)s * m), S.tab.f[(d0 - (S.dim - S.rope)) >> 1], 1.f, &cs, &sn);
      rope_rotate(o0, o1, cs, sn);
    }
  }
  const int64_t slot = (int64_t)b * S.cap + s;
  store_row_pairs(S.dtype, S.dim, S.tail, S.pool + slot * row_bytes(S.dtype, S.dim, S.tail),
                  S.rsc ? S.rsc + slot : nullptr, S.bsc ? S.bsc + slot * (S.dim / 32) : nullptr, o0, o1, active,
                  red);
}

// grid B, block 256
template <bool BF>
__global__ __launch_bounds__(256) void k_cache_state(CacheArgs A) {
  const int b = blockIdx.x;
  const int L = A.len[b];
  const int nb = A.n_new ? max(0, min(A.n_new[b], A.n)) : A.n;
  for (int si = 0; si < A.ns; ++si) {
    const CacheStreamD &S = A.st[si];
    const int nbuf = min(nb, A.span), half = S.dim >> 1;
    const int total = nbuf * half;
    for (int u = threadIdx.x; u < total; u += blockDim.x) {
      const int k = u / half, p = u - k * half;
      const int i = nb - nbuf + k, t = L + i;
      const int64_t pi = ((int64_t)b * A.n + i) * half + p;
      float *br = S.buf + (((int64_t)b * A.span + (t % A.span)) * 2) * S.dim;
      reinterpret_cast<float2 *>(br)[p] = load_pair<BF>(S.c, pi);
      reinterpret_cast<float2 *>(br + S.dim)[p] = load_pair<BF>(S.z, pi);
    }
  }
  __syncthreads();   // every thread has read len[b]
  if (threadIdx.x == 0) {
    const int Ln = L + nb;
    A.len[b] = Ln;
    for (int si = 0; si < A.ns; ++si) {
      const int64_t c = Ln / A.m;
      A.st[si].count[b] = (int32_t)(c < A.st[si].cap ? c : A.st[si].cap);
    }
    if (A.wcap > 0) {
      const int wc = Ln < A.wcap ? Ln : A.wcap;
      A.wcount[b] = wc;
      A.wfirst[b] = Ln - wc;
    }
  }
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

static void fill_stream(CacheStreamD &d, const dsv4_stream &s, const void *c, const void *z) {
  d.dim = s.dim;
  d.rope = s.rope_dim;
  d.dtype = s.pool_dtype;
  d.tail = s.tail;
  d.bias = s.pos_bias;
  d.buf = s.buf;
  d.pool = (uint8_t *)s.pool;
  d.rsc = s.row_scale;
  d.bsc = s.blk_scale;
  d.cap = s.pool_cap;
  d.count = s.count;
  d.c = c;
  d.z = z;
}

int launch_cache_append(const dsv4_cache *C, int n, const int32_t *n_new, const void *kv, const void *kv_c,
                        const void *kv_z, const void *idx_c, const void *idx_z, int in_dtype, hipStream_t st) {
  if (n == 0) return DSV4_OK;
  CacheArgs A{};
  A.B = C->n_seq;
  A.n = n;
  A.m = C->m;
  A.overlap = C->overlap ? 1 : 0;
  A.span = A.overlap ? 2 * C->m : C->m;
  A.theta = C->rope_theta;
  A.pos0 = C->pos0;
  A.len = C->len;
  A.n_new = n_new;
  A.kv = kv;
  A.win = (uint8_t *)C->win;
  A.wsc = C->win_scale;
  A.wdtype = C->win_dtype;
  A.wtail = C->win_tail;
  A.wcap = C->win_cap;
  A.wdim = C->win_dim;
  A.wrope = C->win_rope_dim;
  A.wtab = rope_table(C->rope_theta, A.wrope);
  A.wcount = C->win_count;
  A.wfirst = C->win_first;
  A.nwi = C->win_cap > 0 ? (n < C->win_cap ? n : C->win_cap) : 0;
  A.nei = (n + C->m - 1) / C->m;
  A.ns = 1;
  fill_stream(A.st[0], C->kv, kv_c, kv_z);
  A.st[0].tab = rope_table(C->rope_theta, A.st[0].rope);
  if (C->idx.dim > 0) {
    fill_stream(A.st[1], C->idx, idx_c, idx_z);
    A.st[1].tab = rope_table(C->rope_theta, A.st[1].rope);
    A.ns = 2;
  }
  const bool bf = in_dtype == DSV4_BF16;
  const int64_t items = (int64_t)A.nwi + (int64_t)A.ns * A.nei;
  dim3 g1((unsigned)items, (unsigned)A.B), blk(256);
  if (bf) hipLaunchKernelGGL(k_cache_write<true>, g1, blk, 0, st, A);
  else hipLaunchKernelGGL(k_cache_write<false>, g1, blk, 0, st, A);
  int rc = check_launch("k_cache_write");
  if (rc) return rc;
  dim3 g2((unsigned)A.B);
  if (bf) hipLaunchKernelGGL(k_cache_state<true>, g2, blk, 0, st, A);
  else hipLaunchKernelGGL(k_cache_state<false>, g2, blk, 0, st, A);
  return check_launch("k_cache_state");
}

}  // namespace dsv4host
