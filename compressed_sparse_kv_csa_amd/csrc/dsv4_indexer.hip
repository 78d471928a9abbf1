// dsv4_indexer.hip -- Lightning Indexer scoring and per-query top-k for gfx950.
//
// HF DeepSeek-V4 page, "Hybrid attention": the indexer scores each query
// against the compressed pool and keeps the top index_topk blocks;
// "Attention mask layout": a query sees entry s only once its window closed
// (s < (t+1)/m) and unused slots carry the -1 sentinel.  insight.ai.kr: the
// scores are ReLU multi-head dot products; MarkTechPost: the query/key path is
// MXFP4.
//
//   I(r, s) = score_scale * sum_h w[r,h] * max(0, q_idx[r,h,:] . k_pool[b,s,:])
//
// Kernels
//   k_index_scores_mfma<NHB, KS, FP4>  per (query row, entry chunk): 64 heads
//       as the MFMA M dimension, 16 entries as N, the head dimension as K.
//       bf16: v_mfma_f32_16x16x32_bf16, KS k-steps of 32.  MXFP4: one scaled
//       v_mfma_f32_16x16x128_f8f6f4 per head block, the E8M0 block scales fed
//       straight to the instruction (a lane's 32 k-values are one MX block).
//       Keys are read once, straight from HBM into MFMA registers; the ReLU,
//       the head weights and the head sum run on the accumulators.
//   k_index_scores_f32  scalar fp32 path (small fp32 shapes).
//   k_topk_chunk  rows of up to 16384 visible entries: exact radix select
//       on register-resident order-preserving keys (8-bit digits counted from
//       the top of the keys' own range), ties to the lower index, stable
//       compaction so indices come out ascending.
//   k_rt_hist / k_rt_count / k_rt_emit  longer rows: the exact kk-th largest
//       key from three global histogram passes (11 + 11 + 10 bits) over every
//       chunk of the row, then per-chunk counts and an ordered emission; the
//       same picks, spread over (row, chunk) workgroups.
#include "dsv4_common.h"

#include <algorithm>
#include <map>
#include <mutex>

namespace dsv4 {

struct IdxQ {
  const int32_t *seq, *tok;
  const void *q;          // [T, H, Di] bf16/f32, or [T, H, Di/2] fp4 bytes
  const uint8_t *qscale;  // [T, H, Di/32] (fp4)
  const float *w;         // [T, H]
  int H, Di;
};
struct IdxK {
  const void *data;
  const uint8_t *bscale;  // fp4 block scales [B*stride, Di/32]
  const int32_t *count;
  int64_t stride;
  int m;
};

__device__ __forceinline__ int n_visible(int t, int m, int count) {
  const int n = (t + 1) / m;
  return n < count ? n : count;
}

// order-preserving float -> uint32 key (larger float, larger key)
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float keyf(uint32_t k) {
  const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// -------------------------------------------------------------------- scores (MFMA)
// grid (T, G), block 256 (4 waves).  The row's entries are dealt out in
// super-blocks of 64*EB: workgroup y takes super-blocks y, y + G, y + 2G, ...,
// so at any moment the G workgroups of a row stream one contiguous stretch of
// the pool (DRAM pages stay open).  Wave wv takes the EB 16-entry blocks
// 16*EB*wv + 16*eb of a super-block.  Lane l = 16*g + c:
//   A (query) : head 16*hb + c,   k-slice g   (bf16: dims 32j + 8g .. +8)
//   B (keys)  : entry e0 + c,     k-slice g
//   D         : heads 16*hb + 4g + i (i < 4), entry e0 + c
// The key loads of iteration it+1 are issued before the MFMAs of iteration it
// (two register stages), so each wave keeps 2*EB*16 key rows in flight: the
// decode scan is one pass over a large pool and is bound by how many bytes
// are outstanding, not by the matrix cores.
template <int NHB, int KS, bool FP4, int EB>
__global__ __launch_bounds__(256) void k_index_scores_mfma(IdxQ Q, IdxK K, float scale, uint32_t *hzero,
                                                           int hwords, float *__restrict__ scores, int64_t ld) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  // clear this row's top-k histograms (when the radix passes follow)
  if (hzero && blockIdx.y == 0)
    for (int i = threadIdx.x; i < hwords; i += 256) hzero[(int64_t)r * hwords + i] = 0u;
  const int b = Q.seq[r];
  const int hi = n_visible(Q.tok[r], K.m, K.count[b]);
  constexpr int STEP = 64 * EB;   // entries per super-block
  if ((int64_t)blockIdx.y * STEP >= hi) return;
  const int H = Q.H, Di = Q.Di;

  // query operand and head weights in registers
  bf16x8 qb[NHB][FP4 ? 1 : KS];
  i32x8 qf[NHB];
  int qs[NHB];
  float wt[NHB][4];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const int h = 16 * hb + c;
    if constexpr (FP4) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>((const uint8_t *)Q.q + ((int64_t)r * H + h) * (Di / 2) + 16 * g);
      qf[hb] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      qs[hb] = Q.qscale[((int64_t)r * H + h) * (Di / 32) + g];
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j)
        qb[hb][j] = *reinterpret_cast<const bf16x8 *>((const uint16_t *)Q.q + ((int64_t)r * H + h) * Di + 32 * j + 8 * g);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) wt[hb][i] = Q.w[(int64_t)r * H + 16 * hb + 4 * g + i];
  }

  struct Frag {
    bf16x8 kb[EB][FP4 ? 1 : KS];
    u32x4 kf[EB];
    int ks[EB];
  };
  const int64_t kbase = (int64_t)b * K.stride;
  auto load = [&](int e0, Frag &f) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      const int e = min(e0 + 16 * eb + c, hi - 1);   // clamp: lanes past the end re-read a valid row
      const int64_t row = kbase + e;
      if constexpr (FP4) {
        f.kf[eb] = *reinterpret_cast<const u32x4 *>((const uint8_t *)K.data + row * (Di / 2) + 16 * g);
        f.ks[eb] = K.bscale[row * (Di / 32) + g];
      } else {
#pragma unroll
        for (int j = 0; j < KS; ++j)
          f.kb[eb][j] = *reinterpret_cast<const bf16x8 *>((const uint16_t *)K.data + row * Di + 32 * j + 8 * g);
      }
    }
  };
  auto comp = [&](int e0, const Frag &f) {
#pragma unroll
    for (int eb = 0; eb < EB; ++eb) {
      float s = 0.f;
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (FP4) {
          const i32x8 kb = i32x8{(int)f.kf[eb].x, (int)f.kf[eb].y, (int)f.kf[eb].z, (int)f.kf[eb].w, 0, 0, 0, 0};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[hb], kb, acc, 4, 4, 0, qs[hb], 0, f.ks[eb]);
        } else {
#pragma unroll
          for (int j = 0; j < KS; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[hb][j], f.kb[eb][j], acc, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(wt[hb][i], relu_f(acc[i]), s);
      }
      // sum over the four lane groups (heads 4g..4g+3 of every head block)
      s = rows_sum(s);
      const int e = e0 + 16 * eb + c;
      if (g == 0 && e < hi) scores[(int64_t)r * ld + e] = s * scale;
    }
  };
  const int gstride = (int)gridDim.y * STEP;
  Frag f0, f1;
  int e0 = (int)blockIdx.y * STEP + 16 * EB * wv;
  if (e0 < hi) load(e0, f0);
  for (; e0 < hi; e0 += 2 * gstride) {
    const int e1 = e0 + gstride;
    if (e1 < hi) load(e1, f1);
    comp(e0, f0);
    if (e1 >= hi) break;
    if (e1 + gstride < hi) load(e1 + gstride, f0);
    comp(e1, f1);
  }
}

// -------------------------------------------------------------------- scores, many queries (MFMA)
// k_index_scores_q8<NHB, QPW>: prefill form.  One workgroup scores 4*QPW query
// rows (QPW per wave) against 64-entry key tiles staged once in LDS, so each key
// is read from L2 once per 4*QPW queries.  Same MFMA mapping as above (heads =
// M, entries = N, head dimension = K); queries of the group that belong to
// different sequences are handled one sequence at a time.  QPW = 1 keeps the
// query operand at 64 VGPRs, which leaves room for three waves per SIMD so the
// ReLU / weighting VALU work of one wave overlaps the MFMAs of another.
template <int NHB, int QPW>
__global__ __launch_bounds__(256) void k_index_scores_q8(IdxQ Q, IdxK K, float scale, int T,
                                                         float *__restrict__ scores, int64_t ld) {
  constexpr int KS = 4;          // head dim 128 = 4 k-steps of 32
  constexpr int DI = 128;
  constexpr int KP = DI + 8;     // LDS row pitch (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][64 * KP];
  constexpr int QG = 4 * QPW;   // queries per workgroup
  __shared__ int sh_b[QG], sh_n[QG];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int r0 = (gridDim.x - 1 - blockIdx.x) * QG;   // later (longer) rows first
  const int H = Q.H;
  if (tid < QG) {
    const int r = r0 + tid;
    sh_b[tid] = r < T ? Q.seq[r] : -1;
    sh_n[tid] = r < T ? n_visible(Q.tok[r], K.m, K.count[Q.seq[r]]) : 0;
  }
  // this wave's two queries: operands and weights in registers
  bf16x8 qa[QPW][NHB][KS];
  float wt[QPW][NHB][4];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int r = min(r0 + QPW * wv + qq, T - 1);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int h = 16 * hb + c;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        qa[qq][hb][j] = *reinterpret_cast<const bf16x8 *>((const uint16_t *)Q.q + ((int64_t)r * H + h) * DI + 32 * j + 8 * g);
#pragma unroll
      for (int i = 0; i < 4; ++i) wt[qq][hb][i] = Q.w[(int64_t)r * H + 16 * hb + 4 * g + i];
    }
  }
  // the query loads must be complete before the tile loop: otherwise the
  // compiler's first-use wait inside the loop (vmcnt counts in order) also
  // waits for the next tile's key loads on every iteration
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  __syncthreads();
  for (int sgi = 0; sgi < QG; ++sgi) {
    const int b = sh_b[sgi];
    if (b < 0) break;
    bool seen = false;
    for (int k = 0; k < sgi; ++k) seen |= sh_b[k] == b;
    if (seen) continue;
    int nmax = 0;
    for (int k = 0; k < QG; ++k)
      if (sh_b[k] == b) nmax = max(nmax, sh_n[k]);
    int nq[QPW];
    bool mine[QPW];
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
      mine[qq] = sh_b[QPW * wv + qq] == b;
      nq[qq] = mine[qq] ? sh_n[QPW * wv + qq] : 0;
    }
    const int ntile = (nmax + 63) / 64;
    const uint16_t *kbase = (const uint16_t *)K.data + (int64_t)b * K.stride * DI;
    // staging: thread moves 16 B chunks it = tid + 256 k (k < 4) of the 64 x 128 tile
    auto load = [&](int tile, u32x4 *v) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int it = tid + 256 * k, row = it >> 4, ch = it & 15;
        const int e = min(64 * tile + row, nmax - 1);
        v[k] = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)e * DI + 8 * ch);
      }
    };
    auto store = [&](int buf, const u32x4 *v) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int it = tid + 256 * k, row = it >> 4, ch = it & 15;
        *reinterpret_cast<u32x4 *>(&kt[buf][row * KP + 8 * ch]) = v[k];
      }
    };
    u32x4 stg[4];
    if (ntile > 0) {
      load(0, stg);
      store(0, stg);
    }
    __syncthreads();
    for (int tile = 0; tile < ntile; ++tile) {
      const int buf = tile & 1;
      if (tile + 1 < ntile) load(tile + 1, stg);
      // per-lane partial sums of the tile's 4 entry blocks x 2 queries; the
      // cross-lane head sums run afterwards, all eight together
      float sacc[QPW][4];
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) {
        const int e0 = 64 * tile + 16 * eb;
        bf16x8 kb[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j)
          kb[j] = *reinterpret_cast<const bf16x8 *>(&kt[buf][(16 * eb + c) * KP + 32 * j + 8 * g]);
#pragma unroll
        for (int qq = 0; qq < QPW; ++qq) {
          sacc[qq][eb] = 0.f;
          if (!mine[qq] || e0 >= nq[qq]) continue;   // wave-uniform
          // NHB independent accumulation chains, interleaved k-step by k-step
          f32x4 acc[NHB];
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb)
              acc[hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qq][hb][j], kb[j], acc[hb], 0, 0, 0);
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[qq][eb] = fmaf(wt[qq][hb][i], relu_f(acc[hb][i]), sacc[qq][eb]);
        }
      }
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq)
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) sacc[qq][eb] = rows_sum(sacc[qq][eb]);
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        if (!mine[qq] || g != 0) continue;
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
          const int e = 64 * tile + 16 * eb + c;
          if (e < nq[qq]) scores[(int64_t)(r0 + QPW * wv + qq) * ld + e] = sacc[qq][eb] * scale;
        }
      }
      if (tile + 1 < ntile) store(buf ^ 1, stg);
      __syncthreads();
    }
  }
}

// -------------------------------------------------------------------- scores (fp32 VALU)
// grid (T, n_chunks), block 256: one thread per entry, the query in LDS.
__global__ __launch_bounds__(256) void k_index_scores_f32(IdxQ Q, IdxK K, float scale, int chunk,
                                                          float *__restrict__ scores, int64_t ld) {
  extern __shared__ float qsh[];   // [H*Di] then w[H]
  const int r = blockIdx.x;
  const int b = Q.seq[r];
  const int n = n_visible(Q.tok[r], K.m, K.count[b]);
  const int lo = blockIdx.y * chunk;
  const int hi = min(n, lo + chunk);
  if (lo >= hi) return;
  const int H = Q.H, Di = Q.Di;
  const float *q = (const float *)Q.q + (int64_t)r * H * Di;
  for (int i = threadIdx.x; i < H * Di; i += blockDim.x) qsh[i] = q[i];
  for (int i = threadIdx.x; i < H; i += blockDim.x) qsh[H * Di + i] = Q.w[(int64_t)r * H + i];
  __syncthreads();
  for (int e = lo + threadIdx.x; e < hi; e += blockDim.x) {
    const float *k = (const float *)K.data + ((int64_t)b * K.stride + e) * Di;
    float s = 0.f;
    for (int h = 0; h < H; ++h) {
      float d = 0.f;
      for (int i = 0; i < Di; ++i) d = fmaf(qsh[h * Di + i], k[i], d);
      s = fmaf(qsh[H * Di + h], fmaxf(d, 0.f), s);
    }
    scores[(int64_t)r * ld + e] = s * scale;
  }
}

// -------------------------------------------------------------------- block top-k
// One workgroup of 256 threads selects the kk largest of up to 256*KPT keys
// held in registers: thread t holds positions 4*(t + 256*(j/4)) + j%4, so a
// row of scores loads as coalesced 16-byte vectors.  Keys are order-preserving
// images of the scores (0 = empty).  Exact and deterministic:
//   1. the keys are shifted to k - kmin + 1 so their significant bits start
//      at the top of the block's own range;
//   2. radix select, 8-bit digits from the top: a 256-bin LDS histogram of the
//      keys still matching the chosen prefix, a block scan over the bins in
//      descending order, and the bin holding the want-th largest becomes the
//      next prefix; it stops once the whole boundary group is taken or every
//      bit is resolved;
//   3. equal keys at the boundary are taken lowest position first (a bitmap
//      of the boundary group and a prefix popcount give each its rank);
//   4. the selection is a bitmap over positions; its prefix popcount is every
//      selected key's output slot, so the output comes out in ascending
//      position order with no sort.
struct TkLds {
  uint32_t hist[2][256];
  uint32_t sh[32];
  uint32_t bm[512];     // bitmap over positions (256*KPT/32 words)
  uint32_t wpre[512];   // exclusive prefix popcount of bm per word
};

__device__ __forceinline__ int tk_pos(int j) { return 4 * ((int)threadIdx.x + 256 * (j >> 2)) + (j & 3); }

// Exclusive scan of one value per thread over the 256 threads (one barrier;
// sh4 must not be reused before two more barriers).
__device__ __forceinline__ uint32_t tk_scan(uint32_t v, uint32_t *sh4, uint32_t *total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  if (lane == 63) sh4[wv] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    base += i < wv ? sh4[i] : 0u;
    tot += sh4[i];
  }
  *total = tot;
  return base + inc - v;
}

// L.bm -> L.wpre (nw words); ends with a barrier.
__device__ __forceinline__ void tk_word_prefix(TkLds &L, int nw, uint32_t *sh4) {
  const int per = (nw + 255) / 256, w0 = per * (int)threadIdx.x;
  uint32_t c = 0;
  for (int q = 0; q < per; ++q)
    if (w0 + q < nw) c += __popc(L.bm[w0 + q]);
  uint32_t tot;
  uint32_t run = tk_scan(c, sh4, &tot);
  for (int q = 0; q < per; ++q)
    if (w0 + q < nw) {
      L.wpre[w0 + q] = run;
      run += __popc(L.bm[w0 + q]);
    }
  __syncthreads();
}

__device__ __forceinline__ uint32_t tk_rank(const TkLds &L, int pos) {
  const int w = pos >> 5, bit = pos & 31;
  return L.wpre[w] + __popc(L.bm[w] & ((1u << bit) - 1u));
}

// Select the kk (>= 1) largest non-empty keys; emit(rank, j, key) for each,
// ranks 0..kk-1 in ascending position order.  There must be at least kk
// non-empty keys.
template <int KPT, class Emit>
__device__ void tk_select(uint32_t (&k)[KPT], int kk, TkLds &L, Emit emit) {
  static_assert(KPT % 4 == 0 && KPT <= 64, "keys per thread");
  constexpr int NW = 8 * KPT;   // bitmap words
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  // 1. range of the non-empty keys
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (k[j]) lo = min(lo, k[j]);
    hi = max(hi, k[j]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
  }
  if (lane == 0) {
    L.sh[4 + wv] = lo;
    L.sh[8 + wv] = hi;
  }
  if (tid == 0) {   // the selection if no bin matched (kk beyond the non-empty keys)
    L.sh[0] = 0u;
    L.sh[1] = (uint32_t)kk;
    L.sh[2] = 0u;
  }
  L.hist[0][tid] = 0u;
  for (int w = tid; w < NW; w += 256) L.bm[w] = 0u;
  __syncthreads();
  const uint32_t kmin = min(min(L.sh[4], L.sh[5]), min(L.sh[6], L.sh[7]));
  const uint32_t kmax = max(max(L.sh[8], L.sh[9]), max(L.sh[10], L.sh[11]));
#pragma unroll
  for (int j = 0; j < KPT; ++j) k[j] = k[j] ? k[j] - kmin + 1u : 0u;
  const uint32_t span = kmax - kmin + 1u;
  // 2. radix select
  int hb = 32 - __clz(span);
  uint32_t prefix = 0u, mask = 0u, want = (uint32_t)kk, grp = 0u;
  for (int p = 0; hb > 0; ++p) {
    const int w = hb >= 8 ? 8 : hb, shift = hb - w;
    const uint32_t dm = (1u << w) - 1u;
    uint32_t *H = L.hist[p & 1];
    L.hist[(p + 1) & 1][tid] = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t x = k[j];
      if (x && (x & mask) == prefix) atomicAdd(&H[(x >> shift) & dm], 1u);
    }
    __syncthreads();
    const int bin = 255 - tid;   // thread order = descending bins
    const uint32_t v = H[bin];
    uint32_t tot;
    const uint32_t above = tk_scan(v, L.sh + 12 + 4 * (p % 3), &tot);
    if (above < want && want <= above + v) {
      L.sh[0] = prefix | ((uint32_t)bin << shift);
      L.sh[1] = want - above;
      L.sh[2] = v;
    }
    __syncthreads();
    prefix = L.sh[0];
    want = L.sh[1];
    grp = L.sh[2];
    mask |= dm << shift;
    hb = shift;
    if (grp == want) break;   // the whole boundary group is taken
  }
  // Positions 4*(tid + 256q) + e (e < 4) of a thread share bitmap word
  // (tid + 256q) >> 3, bits 4*(tid & 7) + e: one atomic per group of four, and
  // the rank lookups load each word once.
  const int sh4 = 4 * (tid & 7);
  // 3. ties at the boundary: lowest positions first
  uint64_t take_eq = ~0ull;
  if (grp != want) {
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      uint32_t m4 = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = k[4 * q + e];
        m4 |= (x && (x & mask) == prefix) ? 1u << e : 0u;
      }
      if (m4) atomicOr(&L.bm[(tid + 256 * q) >> 3], m4 << sh4);
    }
    __syncthreads();
    tk_word_prefix(L, NW, L.sh + 24);
    take_eq = 0ull;
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      const int w = (tid + 256 * q) >> 3;
      const uint32_t base = L.wpre[w], bits = L.bm[w];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = k[4 * q + e];
        if (x && (x & mask) == prefix && base + __popc(bits & ((1u << (sh4 + e)) - 1u)) < want)
          take_eq |= 1ull << (4 * q + e);
      }
    }
    __syncthreads();
    for (int w = tid; w < NW; w += 256) L.bm[w] = 0u;
    __syncthreads();
  }
  // 4. selection bitmap -> ranks
  uint64_t selm = 0ull;
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    uint32_t m4 = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * q + e;
      const uint32_t x = k[j];
      const uint32_t xm = x & mask;
      if (x && (xm > prefix || (xm == prefix && ((take_eq >> j) & 1ull)))) {
        m4 |= 1u << e;
        selm |= 1ull << j;
      }
    }
    if (m4) atomicOr(&L.bm[(tid + 256 * q) >> 3], m4 << sh4);
  }
  __syncthreads();
  tk_word_prefix(L, NW, L.sh + 28);
  uint32_t wbits[KPT / 4], wbase[KPT / 4];
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    const int w = (tid + 256 * q) >> 3;
    wbits[q] = L.bm[w];
    wbase[q] = L.wpre[w];
  }
#pragma unroll
  for (int j = 0; j < KPT; ++j)
    if ((selm >> j) & 1ull) {
      const uint32_t rank = wbase[j >> 2] + __popc(wbits[j >> 2] & ((1u << (sh4 + (j & 3))) - 1u));
      if (rank < (uint32_t)kk) emit((int)rank, j, k[j] + kmin - 1u);
    }
}

// grid (T), 256 threads: rows of at most 256*KPT visible entries, selected in
// registers; writes the final idx/score rows.
template <int KPT>
__global__ __launch_bounds__(256) void k_topk_chunk(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                    const int32_t *__restrict__ count, int m,
                                                    const float *__restrict__ scores, int64_t ld, int topk,
                                                    int32_t *__restrict__ idx_out, float *__restrict__ score_out) {
  __shared__ TkLds L;
  const int r = gridDim.x - 1 - blockIdx.x;   // long rows first
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int kk = min(topk, n);
  int32_t *io = idx_out + (int64_t)r * topk;
  float *so = score_out ? score_out + (int64_t)r * topk : nullptr;
  auto emit = [&](int rank, int pos, uint32_t key) {
    io[rank] = pos;
    if (so) so[rank] = keyf(key);
  };
  if (kk == n) {   // everything visible is taken, in order
    for (int j = threadIdx.x; j < n; j += 256) emit(j, j, fkey(scores[(int64_t)r * ld + j]));
  } else {
    uint32_t k[KPT];
    const float *src = scores + (int64_t)r * ld;
    const bool vec = ((((int64_t)r * ld) & 3) == 0) && (((uintptr_t)scores & 15) == 0);
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      const int p = 4 * ((int)threadIdx.x + 256 * q);
      if (vec && p + 3 < n) {
        const f32x4 v = *reinterpret_cast<const f32x4 *>(src + p);
        k[4 * q] = fkey(v[0]);
        k[4 * q + 1] = fkey(v[1]);
        k[4 * q + 2] = fkey(v[2]);
        k[4 * q + 3] = fkey(v[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) k[4 * q + e] = p + e < n ? fkey(src[p + e]) : 0u;
      }
    }
    tk_select<KPT>(k, kk, L, [&](int rank, int j, uint32_t key) { emit(rank, tk_pos(j), key); });
  }
  for (int j = kk + (int)threadIdx.x; j < topk; j += 256) {
    io[j] = -1;
    if (so) so[j] = -INFINITY;
  }
}

// -------------------------------------------------------------------- long rows: radix threshold
// Rows longer than one workgroup's 16384 register-resident keys (decode over
// long pools) are selected by finding the exact kk-th largest key t* of the
// row with three histogram passes over all of the row's chunks (11, 11 and 10
// key bits, global atomic histograms), then counting, per chunk of 4096 keys,
// the keys above t* and equal to t*, and emitting: every key above t*, and the
// lowest-position keys equal to t* up to kk.  Every pass runs one workgroup
// per (row, chunk), so a few long rows still spread over the whole GPU; the
// picks come out in ascending position order (per-chunk prefix counts), with
// the same result as the register-resident select.
constexpr int kRtChunk = 4096;   // keys per workgroup: 16 per thread
constexpr int kRtBins = 2048;

struct RtHist {                   // per row
  uint32_t h[3][kRtBins];
  uint32_t st[2][4];              // prefix, above, want after levels 1 and 2
};

__device__ __forceinline__ int rt_pos(int j) { return 4 * ((int)threadIdx.x + 256 * (j >> 2)) + (j & 3); }

// keys of chunk c of row r (0 = no entry)
__device__ __forceinline__ void rt_load(const float *scores, int64_t ld, int r, int lo, int n, uint32_t (&k)[16]) {
  const float *src = scores + (int64_t)r * ld + lo;
  const bool vec = ((((int64_t)r * ld + lo) & 3) == 0) && (((uintptr_t)scores & 15) == 0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int p = 4 * ((int)threadIdx.x + 256 * q);
    if (vec && lo + p + 3 < n) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(src + p);
#pragma unroll
      for (int e = 0; e < 4; ++e) k[4 * q + e] = fkey(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) k[4 * q + e] = lo + p + e < n ? fkey(src[p + e]) : 0u;
    }
  }
}

// Bin of histogram `h` (nb bins) holding the want-th largest key: returns the
// bin and, in *above, the count of keys in higher bins.  Block-wide; uses sh
// (at least 8 words) and ends with a barrier.
__device__ __forceinline__ int rt_find(const uint32_t *h, int nb, uint32_t want, uint32_t *above, uint32_t *sh) {
  const int per = nb / 256;                      // bins per thread, highest bins to thread 0
  const int top = nb - 1 - per * (int)threadIdx.x;
  uint32_t c[8], tot_t = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    c[i] = i < per ? h[top - i] : 0u;
    tot_t += c[i];
  }
  uint32_t total;
  const uint32_t before = tk_scan(tot_t, sh, &total);   // keys in bins above this thread's
  if (threadIdx.x == 0) {
    sh[4] = 0;
    sh[5] = 0;
  }
  __syncthreads();
  if (before < want && want <= before + tot_t) {
    uint32_t run = before;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < per && run < want && want <= run + c[i]) {
        sh[4] = (uint32_t)(top - i);
        sh[5] = run;
      }
      run += c[i];
    }
  }
  __syncthreads();
  const int bin = (int)sh[4];
  *above = sh[5];
  __syncthreads();
  return bin;
}

// Threshold state after some histogram levels: key prefix, count of keys
// above it and the number still wanted inside it.
struct RtThr {
  uint32_t prefix, above, want;
};
// One more level: the bin of histogram h (nb bins of `bits` bits) that holds
// the want-th largest key under the prefix.
__device__ __forceinline__ RtThr rt_next(const uint32_t *h, int nb, int bits, RtThr t, uint32_t *sh) {
  uint32_t ab;
  const int bin = rt_find(h, nb, t.want, &ab, sh);
  return RtThr{(t.prefix << bits) | (uint32_t)bin, t.above + ab, t.want - ab};
}

// grid (3*kRtBins*T/256), 256 threads: clear the histograms
__global__ __launch_bounds__(256) void k_rt_zero(uint32_t *h, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) h[i] = 0u;
}

// grid (T, n_chunks), 256 threads: histogram level L (0, 1, 2) of the keys
// that match the prefix fixed by the levels before it
template <int L>
__global__ __launch_bounds__(256) void k_rt_hist(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                 const int32_t *__restrict__ count, int m, const float *__restrict__ scores,
                                                 int64_t ld, int topk, RtHist *__restrict__ hist) {
  __shared__ uint32_t lh[kRtBins];
  __shared__ uint32_t sh[8];
  const int r = blockIdx.x, lo = blockIdx.y * kRtChunk;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int kk = min(topk, n);
  if (kk == n || lo >= n) return;   // every entry taken, or nothing here
  RtHist &H = hist[r];
  // the prefix fixed by the levels before this one: level 1 scans level 0's
  // histogram; level 2 starts from the state level 1's chunk 0 recorded
  RtThr t{0u, 0u, (uint32_t)kk};
  if constexpr (L == 1) t = rt_next(H.h[0], kRtBins, 11, t, sh);
  if constexpr (L == 2) t = rt_next(H.h[1], kRtBins, 11, RtThr{H.st[0][0], H.st[0][1], H.st[0][2]}, sh);
  if (L > 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    H.st[L - 1][0] = t.prefix;
    H.st[L - 1][1] = t.above;
    H.st[L - 1][2] = t.want;
  }
  for (int i = threadIdx.x; i < kRtBins; i += 256) lh[i] = 0u;
  uint32_t k[16];
  rt_load(scores, ld, r, lo, n, k);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t key = k[j];
    if (key == 0u) continue;
    if constexpr (L == 0) atomicAdd(&lh[key >> 21], 1u);
    else if constexpr (L == 1) {
      if ((key >> 21) == t.prefix) atomicAdd(&lh[(key >> 10) & 2047u], 1u);
    } else {
      if ((key >> 10) == t.prefix) atomicAdd(&lh[key & 1023u], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < (L == 2 ? 1024 : kRtBins); i += 256)
    if (lh[i]) atomicAdd(&H.h[L][i], lh[i]);
}

// grid (T, n_chunks), 256 threads: keys above t* and equal to t* per chunk;
// chunk 0 also records (t*, keys wanted at t*)
__global__ __launch_bounds__(256) void k_rt_count(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                  const int32_t *__restrict__ count, int m,
                                                  const float *__restrict__ scores, int64_t ld, int topk,
                                                  const RtHist *__restrict__ hist, uint32_t *__restrict__ cnt,
                                                  uint32_t *__restrict__ thr) {
  __shared__ uint32_t sh[8];
  const int r = blockIdx.x, c = blockIdx.y, nch = gridDim.y, lo = c * kRtChunk;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int kk = min(topk, n);
  uint32_t gt = 0, eq = 0;
  if (kk < n && lo < n) {
    const RtHist &H = hist[r];
    const RtThr t = rt_next(H.h[2], 1024, 10, RtThr{H.st[1][0], H.st[1][1], H.st[1][2]}, sh);
    uint32_t k[16];
    rt_load(scores, ld, r, lo, n, k);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      gt += k[j] > t.prefix ? 1u : 0u;
      eq += k[j] == t.prefix ? 1u : 0u;
    }
    uint32_t tot;
    tk_scan(gt, sh, &tot);
    gt = tot;
    __syncthreads();
    tk_scan(eq, sh, &tot);
    eq = tot;
    if (c == 0 && threadIdx.x == 0) {
      thr[2 * r] = t.prefix;
      thr[2 * r + 1] = t.want;
    }
  }
  if (threadIdx.x == 0) {
    cnt[2 * ((int64_t)r * nch + c)] = gt;
    cnt[2 * ((int64_t)r * nch + c) + 1] = eq;
  }
}

// grid (T, n_chunks), 256 threads: write the picks in ascending position order
__global__ __launch_bounds__(256) void k_rt_emit(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                 const int32_t *__restrict__ count, int m,
                                                 const float *__restrict__ scores, int64_t ld, int topk,
                                                 const uint32_t *__restrict__ cnt, const uint32_t *__restrict__ thr,
                                                 int32_t *__restrict__ idx_out, float *__restrict__ score_out) {
  __shared__ uint32_t sh[8];
  const int r = blockIdx.x, c = blockIdx.y, nch = gridDim.y, lo = c * kRtChunk;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int kk = min(topk, n);
  int32_t *io = idx_out + (int64_t)r * topk;
  float *so = score_out ? score_out + (int64_t)r * topk : nullptr;
  if (c == 0)
    for (int j = kk + (int)threadIdx.x; j < topk; j += 256) {
      io[j] = -1;
      if (so) so[j] = -INFINITY;
    }
  if (lo >= n) return;
  if (kk == n) {   // every visible entry is taken, in order
    for (int j = threadIdx.x; j < min(kRtChunk, n - lo); j += 256) {
      io[lo + j] = lo + j;
      if (so) so[lo + j] = scores[(int64_t)r * ld + lo + j];
    }
    return;
  }
  const uint32_t tstar = thr[2 * r], want = thr[2 * r + 1];
  // keys above t* (G) and equal to t* (E) in the chunks before this one; the
  // equal keys are taken in position order up to `want`, so the picks before
  // this chunk are G + min(E, want)
  uint32_t gsum = 0, esum = 0;
  for (int cc = threadIdx.x; cc < c; cc += 256) {
    gsum += cnt[2 * ((int64_t)r * nch + cc)];
    esum += cnt[2 * ((int64_t)r * nch + cc) + 1];
  }
  uint32_t G, E;
  tk_scan(gsum, sh, &G);
  __syncthreads();
  tk_scan(esum, sh, &E);
  __syncthreads();
  const uint32_t sel_before = G + min(E, want);
  const uint32_t quota = E >= want ? 0u : want - E;   // keys equal to t* this chunk may take
  uint32_t k[16];
  rt_load(scores, ld, r, lo, n, k);
  uint32_t eq_run = 0, sel_run = sel_before;
#pragma unroll
  for (int q = 0; q < 4; ++q) {   // position order: q, then thread, then e
    uint32_t ne = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) ne += k[4 * q + e] == tstar ? 1u : 0u;
    uint32_t tot;
    uint32_t er = eq_run + tk_scan(ne, sh, &tot);
    eq_run += tot;
    __syncthreads();
    bool pick[4];
    uint32_t ns = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t key = k[4 * q + e];
      bool p = key > tstar;
      if (key == tstar) {
        p = er < quota;
        ++er;
      }
      pick[e] = p;
      ns += p ? 1u : 0u;
    }
    uint32_t slot = sel_run + tk_scan(ns, sh, &tot);
    sel_run += tot;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (!pick[e]) continue;
      const int pos = lo + 4 * ((int)threadIdx.x + 256 * q) + e;
      io[slot] = pos;
      if (so) so[slot] = keyf(k[4 * q + e]);
      ++slot;
    }
  }
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

// Top-k plan: rows of at most 16384 entries are selected by one workgroup
// each (k_topk_chunk, KPT keys per thread); longer rows by the radix-threshold
// passes over chunks of kRtChunk entries.  Workspace: the score rows, then
// (long rows) the histograms, the per-chunk counts and the thresholds.
struct TopkPlan {
  bool radix;
  int kpt, n_chunks;
  size_t scores_bytes, hist_bytes, cnt_bytes, thr_bytes;
};

static int tk_kpt(int64_t n) {
  int kpt = 4;
  while (kpt < 64 && 256LL * kpt < n) kpt *= 2;
  return kpt;
}

static size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

static TopkPlan plan_topk(int64_t n_rows, int64_t stride, int topk) {
  TopkPlan p{};
  const int64_t st = stride > 0 ? stride : 1;
  p.radix = st > 16384;
  p.kpt = tk_kpt(st);
  p.n_chunks = p.radix ? (int)((st + kRtChunk - 1) / kRtChunk) : 1;
  p.scores_bytes = align256((size_t)n_rows * (size_t)st * 4);
  if (p.radix) {
    p.hist_bytes = align256((size_t)n_rows * sizeof(RtHist));
    p.cnt_bytes = align256((size_t)n_rows * p.n_chunks * 8);
    p.thr_bytes = align256((size_t)n_rows * 8);
  }
  (void)topk;
  return p;
}

size_t index_topk_ws(int64_t n_rows, int64_t stride, int topk) {
  const TopkPlan p = plan_topk(n_rows, stride, topk);
  return p.scores_bytes + p.hist_bytes + p.cnt_bytes + p.thr_bytes + 256;
}

int index_topk_supported(int64_t stride, int topk) {
  // grid.y of the radix passes holds the chunks of a row
  return (stride + kRtChunk - 1) / kRtChunk <= 65535 && topk >= 1;
}

// Workgroups of `kernel` (`block` threads, no dynamic LDS) that the current
// device holds at once; cached per device and kernel.
static int resident_wgs(const void *kernel, int block) {
  static std::mutex mu;
  static std::map<std::pair<int, const void *>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find({dev, kernel});
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess || per_cu < 1) per_cu = 1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 256;
  const int n = per_cu * cus;
  cache[{dev, kernel}] = n;
  return n;
}

int launch_index_topk(const dsv4_queries *q, const void *qv, const uint8_t *qscale, int q_dtype, const float *w,
                      int H, int Di, const dsv4_rows *kp, int m, int topk, float scale, int32_t *idx_out,
                      float *score_out, void *ws, hipStream_t st) {
  const int T = q->n_rows;
  if (T == 0) return DSV4_OK;
  const TopkPlan p = plan_topk(T, kp->seq_stride, topk);
  float *scores = (float *)ws;
  RtHist *hist = p.radix ? (RtHist *)((char *)ws + p.scores_bytes) : nullptr;
  const int hwords = (int)(sizeof(RtHist) / 4);
  bool hist_clear = false;   // the scoring kernel clears the histograms
  IdxQ Q{q->seq, q->tok, qv, qscale, w, H, Di};
  IdxK K{kp->data, kp->blk_scale, kp->count, kp->seq_stride, m};
  const int64_t ld = kp->seq_stride;
  // scoring kernels with one workgroup per (query row, entry chunk)
  typedef void (*ScoreK)(IdxQ, IdxK, float, uint32_t *, int, float *, int64_t);
  ScoreK sk = nullptr;
  int eb = 1;   // entries per wave iteration / 16
  if (q_dtype == DSV4_MXFP4) {
    eb = 4;
    switch (H / 16) {
    case 1: sk = k_index_scores_mfma<1, 1, true, 4>; break;
    case 2: sk = k_index_scores_mfma<2, 1, true, 4>; break;
    case 3: sk = k_index_scores_mfma<3, 1, true, 4>; break;
    default: sk = k_index_scores_mfma<4, 1, true, 4>; break;
    }
  } else if (q_dtype != DSV4_F32 && !(Di == 128 && T >= 2048)) {
    eb = 2;
#define DSV4_IS_H(KS)                                          \
  switch (H / 16) {                                            \
  case 1: sk = k_index_scores_mfma<1, KS, false, 2>; break;    \
  case 2: sk = k_index_scores_mfma<2, KS, false, 2>; break;    \
  case 3: sk = k_index_scores_mfma<3, KS, false, 2>; break;    \
  default: sk = k_index_scores_mfma<4, KS, false, 2>; break;   \
  }
    switch (Di / 32) {
    case 1: DSV4_IS_H(1); break;
    case 2: DSV4_IS_H(2); break;
    case 3: DSV4_IS_H(3); break;
    default: DSV4_IS_H(4); break;
    }
#undef DSV4_IS_H
  }
  if (q_dtype == DSV4_F32) {
    const int sc_chunk = 1024;
    const int sc_chunks = (int)((kp->seq_stride + sc_chunk - 1) / sc_chunk);
    hipLaunchKernelGGL(k_index_scores_f32, dim3(T, sc_chunks > 0 ? sc_chunks : 1), dim3(256),
                       (size_t)(H * Di + H) * 4, st, Q, K, scale, sc_chunk, scores, ld);
  } else if (sk) {
    // the chunk is sized so that the whole grid is resident at once: the scan
    // runs as one wave of workgroups with no partly filled second round
    const int64_t unit = 64LL * eb;   // entries per super-block
    const int64_t blocks = (kp->seq_stride + unit - 1) / unit;
    const int64_t per_row = std::min<int64_t>(std::max<int64_t>(1, resident_wgs((const void *)sk, 256) / T),
                                              std::max<int64_t>(1, blocks));
    hipLaunchKernelGGL(sk, dim3(T, (unsigned)per_row), dim3(256), 0, st, Q, K, scale, (uint32_t *)hist, hwords,
                       scores, ld);
    hist_clear = hist != nullptr;
  } else {
    constexpr int QPW = 1;   // queries per wave (4 per workgroup share each key tile)
    dim3 g8((T + 4 * QPW - 1) / (4 * QPW));
    switch (H / 16) {
    case 1: hipLaunchKernelGGL((k_index_scores_q8<1, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    case 2: hipLaunchKernelGGL((k_index_scores_q8<2, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    case 3: hipLaunchKernelGGL((k_index_scores_q8<3, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    default: hipLaunchKernelGGL((k_index_scores_q8<4, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    }
  }
  int rc = check_launch("k_index_scores");
  if (rc) return rc;
  if (!p.radix) {
#define DSV4_TK1(KPT)                                                                                          \
  hipLaunchKernelGGL((k_topk_chunk<KPT>), dim3(T), dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, \
                     topk, idx_out, score_out)
    switch (p.kpt) {
    case 4: DSV4_TK1(4); break;
    case 8: DSV4_TK1(8); break;
    case 16: DSV4_TK1(16); break;
    case 32: DSV4_TK1(32); break;
    default: DSV4_TK1(64); break;
    }
#undef DSV4_TK1
    return check_launch("k_topk_chunk");
  }
  uint32_t *cnt = (uint32_t *)((char *)hist + p.hist_bytes);
  uint32_t *thr = (uint32_t *)((char *)cnt + p.cnt_bytes);
  if (!hist_clear) {
    const int64_t hw = (int64_t)T * hwords;
    hipLaunchKernelGGL(k_rt_zero, dim3((unsigned)((hw + 255) / 256)), dim3(256), 0, st, (uint32_t *)hist, hw);
  }
  const dim3 g((unsigned)T, (unsigned)p.n_chunks);
  hipLaunchKernelGGL(k_rt_hist<0>, g, dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, topk, hist);
  hipLaunchKernelGGL(k_rt_hist<1>, g, dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, topk, hist);
  hipLaunchKernelGGL(k_rt_hist<2>, g, dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, topk, hist);
  hipLaunchKernelGGL(k_rt_count, g, dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, topk, hist, cnt,
                     thr);
  hipLaunchKernelGGL(k_rt_emit, g, dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, topk, cnt, thr,
                     idx_out, score_out);
  return check_launch("k_rt_emit");
}

}  // namespace dsv4host
