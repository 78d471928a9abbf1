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
//   k_topk_chunk / k_topk_merge  exact radix select (4 x 8-bit digits of an
//       order-preserving key) in LDS, ties to the lower index, stable
//       compaction so indices come out ascending.
#include "dsv4_common.h"

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
// grid (T, n_chunks), block 256 (4 waves).  Wave wv handles entry blocks
// chunk_lo + 16*(wv + 4*it).  Lane l = 16*g + c:
//   A (query) : head 16*hb + c,   k-slice g   (bf16: dims 32j + 8g .. +8)
//   B (keys)  : entry e0 + c,     k-slice g
//   D         : heads 16*hb + 4g + i (i < 4), entry e0 + c
template <int NHB, int KS, bool FP4>
__global__ __launch_bounds__(256) void k_index_scores_mfma(IdxQ Q, IdxK K, float scale, int chunk,
                                                           float *__restrict__ scores, int64_t ld) {
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int b = Q.seq[r];
  const int n = n_visible(Q.tok[r], K.m, K.count[b]);
  const int lo = blockIdx.y * chunk;
  const int hi = min(n, lo + chunk);
  if (lo >= hi) return;
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

  const int64_t kbase = (int64_t)b * K.stride;
  for (int e0 = lo + 16 * wv; e0 < hi; e0 += 64) {
    const int e = min(e0 + c, hi - 1);   // clamp: lanes past the end re-read a valid row
    const int64_t row = kbase + e;
    float s = 0.f;
    if constexpr (FP4) {
      const u32x4 v = *reinterpret_cast<const u32x4 *>((const uint8_t *)K.data + row * (Di / 2) + 16 * g);
      const i32x8 kb = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
      const int ks = K.bscale[row * (Di / 32) + g];
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qf[hb], kb, acc, 4, 4, 0, qs[hb], 0, ks);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(wt[hb][i], fmaxf(acc[i], 0.f), s);
      }
    } else {
      bf16x8 kb[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j)
        kb[j] = *reinterpret_cast<const bf16x8 *>((const uint16_t *)K.data + row * Di + 32 * j + 8 * g);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[hb][j], kb[j], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) s = fmaf(wt[hb][i], fmaxf(acc[i], 0.f), s);
      }
    }
    // sum over the four lane groups (heads 4g..4g+3 of every head block)
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (g == 0 && e0 + c < hi) scores[(int64_t)r * ld + e0 + c] = s * scale;
  }
}

// -------------------------------------------------------------------- scores, many queries (MFMA)
// k_index_scores_q8<NHB>: prefill form.  One workgroup scores 8 query rows
// (2 per wave) against 64-entry key tiles staged once in LDS, so each key is
// read from L2 once per 8 queries instead of once per query.  Same MFMA
// mapping as above (heads = M, entries = N, head dim = K); queries of the group
// that belong to different sequences are handled one sequence at a time.
template <int NHB>
__global__ __launch_bounds__(256) void k_index_scores_q8(IdxQ Q, IdxK K, float scale, int T,
                                                         float *__restrict__ scores, int64_t ld) {
  constexpr int KS = 4;          // head dim 128 = 4 k-steps of 32
  constexpr int DI = 128;
  constexpr int KP = DI + 8;     // LDS row pitch (bf16 elements)
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][64 * KP];
  __shared__ int sh_b[8], sh_n[8];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int r0 = (gridDim.x - 1 - blockIdx.x) * 8;   // later (longer) rows first
  const int H = Q.H;
  if (tid < 8) {
    const int r = r0 + tid;
    sh_b[tid] = r < T ? Q.seq[r] : -1;
    sh_n[tid] = r < T ? n_visible(Q.tok[r], K.m, K.count[Q.seq[r]]) : 0;
  }
  // this wave's two queries: operands and weights in registers
  bf16x8 qa[2][NHB][KS];
  float wt[2][NHB][4];
#pragma unroll
  for (int qq = 0; qq < 2; ++qq) {
    const int r = min(r0 + 2 * wv + qq, T - 1);
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
  __syncthreads();
  for (int sgi = 0; sgi < 8; ++sgi) {
    const int b = sh_b[sgi];
    if (b < 0) break;
    bool seen = false;
    for (int k = 0; k < sgi; ++k) seen |= sh_b[k] == b;
    if (seen) continue;
    int nmax = 0;
    for (int k = 0; k < 8; ++k)
      if (sh_b[k] == b) nmax = max(nmax, sh_n[k]);
    int nq[2];
    bool mine[2];
#pragma unroll
    for (int qq = 0; qq < 2; ++qq) {
      mine[qq] = sh_b[2 * wv + qq] == b;
      nq[qq] = mine[qq] ? sh_n[2 * wv + qq] : 0;
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
#pragma unroll
      for (int eb = 0; eb < 4; ++eb) {
        const int e0 = 64 * tile + 16 * eb;
        bf16x8 kb[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j)
          kb[j] = *reinterpret_cast<const bf16x8 *>(&kt[buf][(16 * eb + c) * KP + 32 * j + 8 * g]);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          if (!mine[qq] || e0 >= nq[qq]) continue;   // wave-uniform
          float sacc = 0.f;
#pragma unroll
          for (int hb = 0; hb < NHB; ++hb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[qq][hb][j], kb[j], acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc = fmaf(wt[qq][hb][i], fmaxf(acc[i], 0.f), sacc);
          }
          sacc += __shfl_xor(sacc, 16, 64);
          sacc += __shfl_xor(sacc, 32, 64);
          if (g == 0 && e0 + c < nq[qq]) scores[(int64_t)(r0 + 2 * wv + qq) * ld + e0 + c] = sacc * scale;
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

// -------------------------------------------------------------------- block radix select
// Block exclusive scan of one value per thread (256 threads).  Returns the
// exclusive prefix; *total receives the block total.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *sh4, uint32_t *total) {
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
    if (i < wv) base += sh4[i];
    tot += sh4[i];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Block of 256 threads.  keys[0..n) in LDS.  Finds the key value T of the
// want-th largest element and how many elements equal to T must be taken
// (the lowest-index ones).  Exact; deterministic.  Three digits of 12, 12 and
// 8 bits: a 4096-bin first digit spreads scores that share a sign and most of
// an exponent, which keeps the LDS histogram atomics mostly conflict-free.
struct SelectResult {
  uint32_t prefix, mask, take_eq;
};

constexpr int kHistBins = 4096;

__device__ SelectResult block_radix_select(const uint32_t *keys, int n, int want, uint32_t *hist,
                                           uint32_t *sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  const int shifts[3] = {20, 8, 0};
  const int widths[3] = {12, 12, 8};
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = shifts[pass];
    const uint32_t dmask = (1u << widths[pass]) - 1u;
    const int nb = 1 << widths[pass];
    for (int i = tid; i < nb; i += 256) hist[i] = 0;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint32_t k = keys[i];
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread owns bins [per*tid, per*tid + per); elements in higher bins
    const int per = nb / 256;
    uint32_t v = 0;
    for (int q = 0; q < per; ++q) v += hist[per * tid + q];
    uint32_t tot;
    const uint32_t before = block_excl_scan(v, sh + 12, &tot);
    uint32_t above = tot - before - v;
    for (int q = per - 1; q >= 0; --q) {
      const uint32_t cq = hist[per * tid + q];
      if (above < (uint32_t)want && (uint32_t)want <= above + cq) {
        sh[0] = prefix | ((uint32_t)(per * tid + q) << shift);
        sh[1] = (uint32_t)want - above;
        sh[2] = cq;
      }
      above += cq;
    }
    __syncthreads();
    prefix = sh[0];
    want = (int)sh[1];
    const uint32_t grp = sh[2];
    mask |= dmask << shift;
    __syncthreads();
    if (grp == (uint32_t)want) break;   // the whole group is taken: no finer digit needed
  }
  return SelectResult{prefix, mask, (uint32_t)want};
}

// Select the top `kk` of keys[0..n) (kk <= n) and write, in ascending position
// order, out_pos[j] = position and out_key[j] = key for j < kk.
__device__ void block_topk_compact(const uint32_t *keys, int n, int kk, uint32_t *hist, uint32_t *sh,
                                   int32_t *out_pos, uint32_t *out_key) {
  const SelectResult sel = block_radix_select(keys, n, kk, hist, sh);
  const int tid = threadIdx.x;
  const int seg = (n + 255) / 256;
  const int a = min(n, tid * seg), bnd = min(n, a + seg);
  uint32_t gt = 0, eq = 0;
  for (int i = a; i < bnd; ++i) {
    const uint32_t k = keys[i] & sel.mask;
    gt += k > sel.prefix;
    eq += k == sel.prefix;
  }
  uint32_t tot;
  const uint32_t eq_before = block_excl_scan(eq, sh + 4, &tot);
  uint32_t eq_take = 0;
  if (eq_before < sel.take_eq) eq_take = min(eq, sel.take_eq - eq_before);
  const uint32_t off = block_excl_scan(gt + eq_take, sh + 8, &tot);
  uint32_t o = off, eq_used = 0;
  for (int i = a; i < bnd; ++i) {
    const uint32_t kf = keys[i];
    const uint32_t k = kf & sel.mask;
    bool take = k > sel.prefix;
    if (!take && k == sel.prefix && eq_used < eq_take) { take = true; ++eq_used; }
    if (take) {
      out_pos[o] = i;
      if (out_key) out_key[o] = kf;
      ++o;
    }
  }
}

// grid (T, n_chunks).  Chunk c covers entries [c*chunk, min(n, (c+1)*chunk)).
// n_chunks == 1: writes the final idx/score rows.  Otherwise writes per-chunk
// candidates (ascending entry order, key 0 in unused slots).
__global__ __launch_bounds__(256) void k_topk_chunk(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                    const int32_t *__restrict__ count, int m,
                                                    const float *__restrict__ scores, int64_t ld, int chunk,
                                                    int topk, int32_t *__restrict__ idx_out,
                                                    float *__restrict__ score_out, uint32_t *__restrict__ cand_key,
                                                    int32_t *__restrict__ cand_idx) {
  extern __shared__ uint32_t smem[];
  uint32_t *keys = smem;                       // [chunk]
  int32_t *pos = (int32_t *)(smem + chunk);    // [topk]
  uint32_t *kout = smem + chunk + topk;        // [topk]
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t sh[16];
  const int r = gridDim.x - 1 - blockIdx.x, cidx = blockIdx.y, nch = gridDim.y;   // long rows first
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int lo = cidx * chunk;
  const int len = max(0, min(n, lo + chunk) - lo);
  const int kk = min(topk, len);
  for (int i = threadIdx.x; i < len; i += 256) keys[i] = fkey(scores[(int64_t)r * ld + lo + i]);
  __syncthreads();
  if (kk > 0) block_topk_compact(keys, len, kk, hist, sh, pos, kout);
  __syncthreads();
  if (nch == 1) {
    for (int j = threadIdx.x; j < topk; j += 256) {
      idx_out[(int64_t)r * topk + j] = j < kk ? lo + pos[j] : -1;
      if (score_out) score_out[(int64_t)r * topk + j] = j < kk ? keyf(kout[j]) : -INFINITY;
    }
  } else {
    const int64_t base = ((int64_t)r * nch + cidx) * topk;
    for (int j = threadIdx.x; j < topk; j += 256) {
      cand_key[base + j] = j < kk ? kout[j] : 0u;
      cand_idx[base + j] = j < kk ? lo + pos[j] : -1;
    }
  }
}

// grid (T).  Merges n_chunks*topk candidates (key 0 = empty) into the final row.
__global__ __launch_bounds__(256) void k_topk_merge(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                    const int32_t *__restrict__ count, int m, int n_chunks,
                                                    int topk, const uint32_t *__restrict__ cand_key,
                                                    const int32_t *__restrict__ cand_idx,
                                                    int32_t *__restrict__ idx_out, float *__restrict__ score_out) {
  extern __shared__ uint32_t smem[];
  const int nc = n_chunks * topk;
  uint32_t *keys = smem;                    // [nc]
  int32_t *pos = (int32_t *)(smem + nc);    // [topk]
  uint32_t *kout = smem + nc + topk;        // [topk]
  __shared__ uint32_t hist[kHistBins];
  __shared__ uint32_t sh[16];
  const int r = blockIdx.x;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int kk = min(topk, n);
  const int64_t base = (int64_t)r * nc;
  for (int i = threadIdx.x; i < nc; i += 256) keys[i] = cand_key[base + i];
  __syncthreads();
  if (kk > 0) block_topk_compact(keys, nc, kk, hist, sh, pos, kout);
  __syncthreads();
  for (int j = threadIdx.x; j < topk; j += 256) {
    idx_out[(int64_t)r * topk + j] = j < kk ? cand_idx[base + pos[j]] : -1;
    if (score_out) score_out[(int64_t)r * topk + j] = j < kk ? keyf(kout[j]) : -INFINITY;
  }
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

// Chunking of the pool for scoring and top-k: the first-stage chunk holds at
// most 16384 keys (64 KB of LDS); the merge stage holds n_chunks*topk keys.
struct TopkPlan {
  int chunk, n_chunks;
  size_t scores_bytes, cand_bytes;
};

static TopkPlan plan_topk(int64_t n_rows, int64_t stride, int topk) {
  TopkPlan p;
  int64_t ch = 4096;
  while (ch < 16384 && ((stride + ch - 1) / ch) * topk > 16384) ch *= 2;
  if (stride <= ch) ch = stride > 0 ? stride : 1;
  p.chunk = (int)ch;
  p.n_chunks = (int)((stride + ch - 1) / ch);
  if (p.n_chunks < 1) p.n_chunks = 1;
  p.scores_bytes = (size_t)n_rows * (size_t)stride * 4;
  p.scores_bytes = (p.scores_bytes + 255) & ~(size_t)255;
  p.cand_bytes = p.n_chunks > 1 ? (size_t)n_rows * p.n_chunks * topk * 8 : 0;
  return p;
}

size_t index_topk_ws(int64_t n_rows, int64_t stride, int topk) {
  const TopkPlan p = plan_topk(n_rows, stride, topk);
  return p.scores_bytes + p.cand_bytes + 256;
}

int index_topk_supported(int64_t stride, int topk) {
  const TopkPlan p = plan_topk(1, stride, topk);
  return (int64_t)p.n_chunks * topk <= 16384 + 0 || p.n_chunks == 1;
}

int launch_index_topk(const dsv4_queries *q, const void *qv, const uint8_t *qscale, int q_dtype, const float *w,
                      int H, int Di, const dsv4_rows *kp, int m, int topk, float scale, int32_t *idx_out,
                      float *score_out, void *ws, hipStream_t st) {
  const int T = q->n_rows;
  if (T == 0) return DSV4_OK;
  const TopkPlan p = plan_topk(T, kp->seq_stride, topk);
  float *scores = (float *)ws;
  uint32_t *cand_key = (uint32_t *)((char *)ws + p.scores_bytes);
  int32_t *cand_idx = (int32_t *)(cand_key + (size_t)T * p.n_chunks * topk);
  IdxQ Q{q->seq, q->tok, qv, qscale, w, H, Di};
  IdxK K{kp->data, kp->blk_scale, kp->count, kp->seq_stride, m};
  const int64_t ld = kp->seq_stride;
  // scoring chunk: 1024 entries per workgroup (16 blocks per wave)
  const int sc_chunk = 1024;
  const int sc_chunks = (int)((kp->seq_stride + sc_chunk - 1) / sc_chunk);
  dim3 sgrid(T, sc_chunks > 0 ? sc_chunks : 1);
  if (q_dtype == DSV4_F32) {
    hipLaunchKernelGGL(k_index_scores_f32, sgrid, dim3(256), (size_t)(H * Di + H) * 4, st, Q, K, scale, sc_chunk,
                       scores, ld);
  } else if (q_dtype == DSV4_MXFP4) {
    switch (H / 16) {
    case 1: hipLaunchKernelGGL((k_index_scores_mfma<1, 1, true>), sgrid, dim3(256), 0, st, Q, K, scale, sc_chunk, scores, ld); break;
    case 2: hipLaunchKernelGGL((k_index_scores_mfma<2, 1, true>), sgrid, dim3(256), 0, st, Q, K, scale, sc_chunk, scores, ld); break;
    case 3: hipLaunchKernelGGL((k_index_scores_mfma<3, 1, true>), sgrid, dim3(256), 0, st, Q, K, scale, sc_chunk, scores, ld); break;
    default: hipLaunchKernelGGL((k_index_scores_mfma<4, 1, true>), sgrid, dim3(256), 0, st, Q, K, scale, sc_chunk, scores, ld); break;
    }
  } else if (Di == 128 && T >= 2048) {
    dim3 g8((T + 7) / 8);
    switch (H / 16) {
    case 1: hipLaunchKernelGGL((k_index_scores_q8<1>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    case 2: hipLaunchKernelGGL((k_index_scores_q8<2>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    case 3: hipLaunchKernelGGL((k_index_scores_q8<3>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    default: hipLaunchKernelGGL((k_index_scores_q8<4>), g8, dim3(256), 0, st, Q, K, scale, T, scores, ld); break;
    }
  } else {
#define DSV4_IS(NHB, KS) hipLaunchKernelGGL((k_index_scores_mfma<NHB, KS, false>), sgrid, dim3(256), 0, st, Q, K, scale, sc_chunk, scores, ld)
#define DSV4_IS_H(KS)                  \
  switch (H / 16) {                    \
  case 1: DSV4_IS(1, KS); break;       \
  case 2: DSV4_IS(2, KS); break;       \
  case 3: DSV4_IS(3, KS); break;       \
  default: DSV4_IS(4, KS); break;      \
  }
    switch (Di / 32) {
    case 1: DSV4_IS_H(1); break;
    case 2: DSV4_IS_H(2); break;
    case 3: DSV4_IS_H(3); break;
    default: DSV4_IS_H(4); break;
    }
#undef DSV4_IS_H
#undef DSV4_IS
  }
  int rc = check_launch("k_index_scores");
  if (rc) return rc;
  const size_t lds1 = ((size_t)p.chunk + 2 * (size_t)topk) * 4;
  hipLaunchKernelGGL(k_topk_chunk, dim3(T, p.n_chunks), dim3(256), lds1, st, q->seq, q->tok, kp->count, m, scores, ld,
                     p.chunk, topk, idx_out, score_out, cand_key, cand_idx);
  rc = check_launch("k_topk_chunk");
  if (rc || p.n_chunks == 1) return rc;
  const size_t lds2 = ((size_t)p.n_chunks * topk + 2 * (size_t)topk) * 4;
  hipLaunchKernelGGL(k_topk_merge, dim3(T), dim3(256), lds2, st, q->seq, q->tok, kp->count, m, p.n_chunks, topk,
                     cand_key, cand_idx, idx_out, score_out);
  return check_launch("k_topk_merge");
}

}  // namespace dsv4host
