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
//   k_rt_cand / k_rt_final  longer rows: a histogram of the top 11 key bits
//       (built while the decode scan stores the scores) bounds the kk-th
//       largest key from below; the keys at or above that bound are
//       compacted in position order, and one workgroup per row selects the
//       exact picks among them (or over the whole row when a chunk's
//       candidates overflow).
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
// are outstanding, not by the matrix cores.  The loop issues loads only: the
// scores are staged in LDS and written out after it (a store in the loop would
// count in the same in-order counter as the loads, and the wait for one stage
// would then also wait for the stores behind it).  A workgroup handles at most
// kScoreStage / (64 EB) - 1 super-blocks (the launcher sizes the grid so).
// With hist0 set (rows that take the long-row top-k) every score is also
// counted in an LDS histogram of its key's top 11 bits, added to the row's
// histogram at the end.
constexpr int kHistBins = 2048;
constexpr int kScoreStage = 4096;   // staged scores per workgroup
template <int NHB, int KS, bool FP4, int EB>
__global__ __launch_bounds__(256) void k_index_scores_mfma(IdxQ Q, IdxK K, float scale, uint32_t *hist0,
                                                           float *__restrict__ scores, int64_t ld) {
  __shared__ uint32_t lh[kHistBins];
  __shared__ float sbuf[kScoreStage];
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int b = Q.seq[r];
  const int hi = n_visible(Q.tok[r], K.m, K.count[b]);
  constexpr int STEP = 64 * EB;   // entries per super-block
  if ((int64_t)blockIdx.y * STEP >= hi) return;
  const int H = Q.H, Di = Q.Di;
  if (hist0) {
    for (int i = threadIdx.x; i < kHistBins; i += 256) lh[i] = 0u;
    __syncthreads();
  }

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
  auto comp = [&](int e0, const Frag &f, int slot) {
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
      if (g == 0) {
        const float v = s * scale;
        sbuf[slot * STEP + 16 * EB * wv + 16 * eb + c] = v;
        if (hist0 && e < hi) atomicAdd(&lh[fkey(v) >> 21], 1u);
      }
    }
  };
  const int gstride = (int)gridDim.y * STEP;
  const int sb_lo = (int)blockIdx.y * STEP;   // this workgroup's first super-block
  const int nsb = (hi - sb_lo + gstride - 1) / gstride;
  Frag f0, f1;
  const int ew = 16 * EB * wv;
  // super-blocks go in pairs (an odd count ends with a stage past the end);
  // the stage loads are unconditional (load() clamps rows past the end to the
  // last one) and the loop has one exit point, so with no branch around a
  // load the compiler's wait before a stage's products leaves the other
  // stage's loads in flight; the scheduling barriers keep that program order
  load(sb_lo + ew, f0);
  load(sb_lo + gstride + ew, f1);
  __builtin_amdgcn_sched_barrier(0);
  for (int k = 0;; k += 2) {
    const int e0 = sb_lo + k * gstride + ew;
    comp(e0, f0, k);
    __builtin_amdgcn_sched_barrier(0);
    load(e0 + 2 * gstride, f0);
    __builtin_amdgcn_sched_barrier(0);
    comp(e0 + gstride, f1, k + 1);
    __builtin_amdgcn_sched_barrier(0);
    load(e0 + 3 * gstride, f1);
    __builtin_amdgcn_sched_barrier(0);
    if (k + 2 >= nsb) break;
  }
  __syncthreads();
  // the staged scores out, super-block by super-block (contiguous entries)
  float *srow = scores + (int64_t)r * ld;
  for (int i = threadIdx.x; i < nsb * STEP; i += 256) {
    const int e = sb_lo + (i / STEP) * gstride + i % STEP;
    if (e < hi) srow[e] = sbuf[i];
  }
  if (hist0) {
    for (int i = threadIdx.x; i < kHistBins; i += 256)
      if (lh[i]) atomicAdd(&hist0[(int64_t)r * kHistBins + i], lh[i]);
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
__global__ __launch_bounds__(256) void k_index_scores_q8(IdxQ Q, IdxK K, float scale, int T, int skip_n,
                                                         float *__restrict__ scores, int64_t ld) {
  constexpr int KS = 4;          // head dim 128 = 4 k-steps of 32
  constexpr int DI = 128;
  constexpr int KP = DI + 16;    // LDS row pitch (bf16 elements; measured against +8 and +24: 151 -> 143 us)
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
    // a row with at most skip_n visible entries takes all of them whatever
    // their scores (skip_n = top-k when no pick scores are wanted): not scored
    const int n = r < T ? n_visible(Q.tok[r], K.m, K.count[Q.seq[r]]) : 0;
    sh_n[tid] = n <= skip_n ? 0 : n;
  }
  // this wave's queries: operands and weights in registers (not loaded for a
  // row that is not scored)
  bf16x8 qa[QPW][NHB][KS];
  float wt[QPW][NHB][4];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int r = min(r0 + QPW * wv + qq, T - 1);
    if (skip_n > 0 && n_visible(Q.tok[r], K.m, K.count[Q.seq[r]]) <= skip_n) {   // wave-uniform
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
        for (int j = 0; j < KS; ++j) qa[qq][hb][j] = bf16x8{};
#pragma unroll
        for (int i = 0; i < 4; ++i) wt[qq][hb][i] = 0.f;
      }
      continue;
    }
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
      // the next tile into LDS before this tile's scores go out: the wait for
      // the staged key loads then leaves the score stores in flight (vmcnt
      // counts stores and loads in issue order; 151 -> 144 us at S = 8192)
      if (tile + 1 < ntile) store(buf ^ 1, stg);
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        if (!mine[qq] || g != 0) continue;
#pragma unroll
        for (int eb = 0; eb < 4; ++eb) {
          const int e = 64 * tile + 16 * eb + c;
          if (e < nq[qq]) scores[(int64_t)(r0 + QPW * wv + qq) * ld + e] = sacc[qq][eb] * scale;
        }
      }
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
// One workgroup of NT threads (128 or 256) selects the kk largest of up to
// NT*KPT keys held in registers: thread t holds positions 4*(t + NT*(j/4)) +
// j%4, so a row of scores loads as coalesced 16-byte vectors.  Short rows take
// 128 threads, so twice as many rows are resident per CU (each step of the
// select waits on a barrier or an LDS round trip, not on the VALU).  Keys are order-preserving
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
  uint32_t bm[512];     // bitmap over positions (NT*KPT/32 words)
  uint32_t wpre[512];   // exclusive prefix popcount of bm per word
};

template <int NT>
__device__ __forceinline__ int tk_pos(int j) { return 4 * ((int)threadIdx.x + NT * (j >> 2)) + (j & 3); }

// Exclusive scan of one value per thread over the NT threads (one barrier;
// sh4 must not be reused before two more barriers).
template <int NT = 256>
__device__ __forceinline__ uint32_t tk_scan(uint32_t v, uint32_t *sh4, uint32_t *total) {
  constexpr int NWV = NT / 64;
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
  for (int i = 0; i < NWV; ++i) {
    base += i < wv ? sh4[i] : 0u;
    tot += sh4[i];
  }
  *total = tot;
  return base + inc - v;
}

// L.bm -> L.wpre (nw words); ends with a barrier.
template <int NT>
__device__ __forceinline__ void tk_word_prefix(TkLds &L, int nw, uint32_t *sh4) {
  const int per = (nw + NT - 1) / NT, w0 = per * (int)threadIdx.x;
  uint32_t c = 0;
  for (int q = 0; q < per; ++q)
    if (w0 + q < nw) c += __popc(L.bm[w0 + q]);
  uint32_t tot;
  uint32_t run = tk_scan<NT>(c, sh4, &tot);
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
template <int KPT, int NT, class Emit>
__device__ void tk_select(uint32_t (&k)[KPT], int kk, TkLds &L, Emit emit) {
  static_assert(KPT % 4 == 0 && KPT <= 64, "keys per thread");
  static_assert(NT == 64 || NT == 128 || NT == 256, "threads per row");
  constexpr int NW = NT * KPT / 32;   // bitmap words
  constexpr int NWV = NT / 64;        // waves
  constexpr int BPT = 256 / NT;       // histogram bins per thread
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
#pragma unroll
  for (int i = 0; i < BPT; ++i) L.hist[0][tid + NT * i] = 0u;
  for (int w = tid; w < NW; w += NT) L.bm[w] = 0u;
  __syncthreads();
  uint32_t kmin = L.sh[4], kmax = L.sh[8];
#pragma unroll
  for (int i = 1; i < NWV; ++i) {
    kmin = min(kmin, L.sh[4 + i]);
    kmax = max(kmax, L.sh[8 + i]);
  }
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
#pragma unroll
    for (int i = 0; i < BPT; ++i) L.hist[(p + 1) & 1][tid + NT * i] = 0u;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const uint32_t x = k[j];
      if (x && (x & mask) == prefix) atomicAdd(&H[(x >> shift) & dm], 1u);
    }
    __syncthreads();
    // thread order = descending bins: thread t holds bins 255 - BPT t - i (i < BPT)
    uint32_t v[BPT], vt = 0u;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      v[i] = H[255 - BPT * tid - i];
      vt += v[i];
    }
    uint32_t tot;
    uint32_t above = tk_scan<NT>(vt, L.sh + 12 + 4 * (p % 3), &tot);
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      if (above < want && want <= above + v[i]) {
        L.sh[0] = prefix | ((uint32_t)(255 - BPT * tid - i) << shift);
        L.sh[1] = want - above;
        L.sh[2] = v[i];
      }
      above += v[i];
    }
    __syncthreads();
    prefix = L.sh[0];
    want = L.sh[1];
    grp = L.sh[2];
    mask |= dm << shift;
    hb = shift;
    if (grp == want) break;   // the whole boundary group is taken
  }
  // Positions 4*(tid + NT q) + e (e < 4) of a thread share bitmap word
  // (tid + NT q) >> 3, bits 4*(tid & 7) + e: one atomic per group of four, and
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
      if (m4) atomicOr(&L.bm[(tid + NT * q) >> 3], m4 << sh4);
    }
    __syncthreads();
    tk_word_prefix<NT>(L, NW, L.sh + 24);
    take_eq = 0ull;
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      const int w = (tid + NT * q) >> 3;
      const uint32_t base = L.wpre[w], bits = L.bm[w];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = k[4 * q + e];
        if (x && (x & mask) == prefix && base + __popc(bits & ((1u << (sh4 + e)) - 1u)) < want)
          take_eq |= 1ull << (4 * q + e);
      }
    }
    __syncthreads();
    for (int w = tid; w < NW; w += NT) L.bm[w] = 0u;
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
    if (m4) atomicOr(&L.bm[(tid + NT * q) >> 3], m4 << sh4);
  }
  __syncthreads();
  tk_word_prefix<NT>(L, NW, L.sh + 28);
  uint32_t wbits[KPT / 4], wbase[KPT / 4];
#pragma unroll
  for (int q = 0; q < KPT / 4; ++q) {
    const int w = (tid + NT * q) >> 3;
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

// grid (T), NT threads: rows of at most NT*KPT visible entries, selected in
// registers; writes the final idx/score rows.
template <int KPT, int NT>
__global__ __launch_bounds__(NT) void k_topk_chunk(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
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
  if (kk == n) {   // everything visible is taken, in order (scores read only for score_out)
    if (so) {
      for (int j = threadIdx.x; j < n; j += NT) emit(j, j, fkey(scores[(int64_t)r * ld + j]));
    } else {
      for (int j = threadIdx.x; j < n; j += NT) io[j] = j;
    }
  } else {
    uint32_t k[KPT];
    const float *src = scores + (int64_t)r * ld;
    const bool vec = ((((int64_t)r * ld) & 3) == 0) && (((uintptr_t)scores & 15) == 0);
#pragma unroll
    for (int q = 0; q < KPT / 4; ++q) {
      const int p = 4 * ((int)threadIdx.x + NT * q);
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
    tk_select<KPT, NT>(k, kk, L, [&](int rank, int j, uint32_t key) { emit(rank, tk_pos<NT>(j), key); });
  }
  for (int j = kk + (int)threadIdx.x; j < topk; j += NT) {
    io[j] = -1;
    if (so) so[j] = -INFINITY;
  }
}

// -------------------------------------------------------------------- long rows: candidates
// Rows longer than one workgroup's 16384 register-resident keys (decode over
// long pools) take three steps:
//   1. a histogram of the top 11 key bits over the whole row (built by the
//      decode scoring kernel as it stores the scores, or by k_rt_hist0);
//   2. k_rt_cand, one workgroup per (row, chunk): the bin b0 holding the
//      kk-th largest key is found from the histogram, and every key at or
//      above b0's lower edge is a candidate; each chunk compacts its
//      candidates in position order into its own slot range (at most cc
//      slots; the true count is recorded).  The candidates hold every key of
//      the top kk, since the histogram counted at least kk keys at or above
//      the edge;
//   3. k_rt_final, one workgroup per row: the candidates above bin b0 are all
//      picked; the keys of bin b0 are refined by two more histogram levels
//      (11 and 10 bits, spread over many bins, so LDS atomics rarely collide)
//      to the exact kk-th largest key t*; the keys above t* and the
//      lowest-position keys equal to t* are written in ascending position
//      order.  A row whose chunk overflowed its slots or that has more than
//      8192 candidates (heavy ties at the edge) is selected by the same
//      workgroup over the whole score row instead: three histogram levels
//      (11, 11, 10 bits), then the ordered emission.
constexpr int kRtChunk = 4096;    // keys per load round: 16 per thread
constexpr int kRtBins = 2048;     // level-0 histogram (top 11 key bits)
constexpr int kCandSlots = 16384; // candidate slots per row (the select's register capacity)
constexpr int kCandMaxChunks = 64;
constexpr int kCandRow = kCandMaxChunks + 4;   // per row: chunk counts, then b0 and the count above it

// keys of positions lo + 4*(t + 256q) + e (q, e < 4) of row r (0 = no entry at
// or past n)
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

// grid ((n + 255) / 256), 256 threads: clear n words
__global__ __launch_bounds__(256) void k_rt_zero(uint32_t *h, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) h[i] = 0u;
}

// Add the keys of positions [lo, hi) of row r (a multiple of kRtChunk apart)
// to the LDS histogram lh: level 0 all keys by their top 11 bits; level 1 the
// keys whose top 11 bits equal the prefix, by the next 11; level 2 the keys
// whose top 22 bits equal it, by the last 10.
template <int L>
__device__ __forceinline__ void rt_hist_range(const float *scores, int64_t ld, int r, int lo, int hi, uint32_t prefix,
                                              uint32_t *lh) {
  for (int base = lo; base < hi; base += kRtChunk) {
    uint32_t k[16];
    rt_load(scores, ld, r, base, hi, k);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t key = k[j];
      if (key == 0u) continue;
      if constexpr (L == 0) atomicAdd(&lh[key >> 21], 1u);
      else if constexpr (L == 1) {
        if ((key >> 21) == prefix) atomicAdd(&lh[(key >> 10) & 2047u], 1u);
      } else {
        if ((key >> 10) == prefix) atomicAdd(&lh[key & 1023u], 1u);
      }
    }
  }
}

// grid (T, n_chunks), 256 threads: the level-0 histogram of rows whose scores
// came from a kernel that does not build it (many-query and fp32 scoring)
__global__ __launch_bounds__(256) void k_rt_hist0(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                  const int32_t *__restrict__ count, int m,
                                                  const float *__restrict__ scores, int64_t ld, int topk,
                                                  uint32_t *__restrict__ hist0) {
  __shared__ uint32_t lh[kRtBins];
  const int r = blockIdx.x, lo = blockIdx.y * kRtChunk;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  if (min(topk, n) == n || lo >= n) return;   // every entry taken, or nothing here
  for (int i = threadIdx.x; i < kRtBins; i += 256) lh[i] = 0u;
  __syncthreads();
  rt_hist_range<0>(scores, ld, r, lo, min(n, lo + kRtChunk), 0u, lh);
  __syncthreads();
  for (int i = threadIdx.x; i < kRtBins; i += 256)
    if (lh[i]) atomicAdd(&hist0[(int64_t)r * kRtBins + i], lh[i]);
}

// One workgroup selects the kk largest keys of row r (n entries) straight
// from the score row: three histogram levels to the exact kk-th largest key
// t*, then every key above t* and the lowest-position keys equal to t*, in
// ascending position order.
__device__ __forceinline__ void rt_row_select(const float *scores, int64_t ld, int r, int n, int kk, int32_t *io, float *so,
                              uint32_t *lh, uint32_t *sh) {
  RtThr t{0u, 0u, (uint32_t)kk};
#pragma unroll
  for (int L = 0; L < 3; ++L) {
    for (int i = threadIdx.x; i < kRtBins; i += 256) lh[i] = 0u;
    __syncthreads();
    if (L == 0) rt_hist_range<0>(scores, ld, r, 0, n, 0u, lh);
    else if (L == 1) rt_hist_range<1>(scores, ld, r, 0, n, t.prefix, lh);
    else rt_hist_range<2>(scores, ld, r, 0, n, t.prefix, lh);
    __syncthreads();
    t = rt_next(lh, L == 2 ? 1024 : kRtBins, L == 2 ? 10 : 11, t, sh);
  }
  const uint32_t tstar = t.prefix, quota = t.want;
  uint32_t eq_run = 0, sel_run = 0;
  for (int base = 0; base < n; base += kRtChunk) {
    uint32_t k[16];
    rt_load(scores, ld, r, base, n, k);
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
        io[slot] = base + 4 * ((int)threadIdx.x + 256 * q) + e;
        if (so) so[slot] = keyf(k[4 * q + e]);
        ++slot;
      }
    }
  }
}

constexpr int kRtMapWords = 256;   // bitmap words over at most 8192 candidates
struct RtFinalLds {
  uint32_t soff[kCandMaxChunks + 1];
  uint32_t lh[kRtBins];
  uint32_t bm[2][kRtMapWords];   // candidate bitmaps in position order: keys equal to t*, picks
  uint32_t wpre[kRtMapWords];    // exclusive prefix popcount per bitmap word
  uint32_t sh[8];
  int over;
};

// bm[0, nw) -> wpre (nw <= 256 words); ends with a barrier
__device__ __forceinline__ void rt_word_prefix(const uint32_t *bm, uint32_t *wpre, int nw, uint32_t *sh4) {
  const int w = (int)threadIdx.x;
  const uint32_t c = w < nw ? (uint32_t)__popc(bm[w]) : 0u;
  uint32_t tot;
  const uint32_t run = tk_scan(c, sh4, &tot);
  if (w < nw) wpre[w] = run;
  __syncthreads();
}

// The kk largest of the row's M candidates (candidate i in position order is
// slot c*cc + (i - off[c]) of the chunk c with off[c] <= i < off[c + 1]).
// Every candidate above the level-0 bin b0 is taken (`above` of them); the
// keys of bin b0 are refined by two more histogram levels (the next 11 and
// the last 10 key bits) to the exact kk-th largest key t*; then the keys above
// t* and the first `want` keys equal to t* are written in position order.
// Candidate i (the row's candidates concatenated chunk by chunk, which is
// position order) goes to thread i mod 256, so each wave's key and position
// loads read consecutive slots; its chunk comes from a search of the offsets
// in LDS with no branch (off[c] = M for every chunk c >= nch), and every load
// is issued unconditionally (the slot clamped into the row's range, the value
// dropped for i >= M).  Output slots come from bitmaps over i and their
// prefix popcounts: the picks', and (only when t* has more equal keys than
// are wanted) the equal keys' to rank them.
template <int P>
__device__ __forceinline__ void rt_cands_select(const uint32_t *rk, const int32_t *rp, int nch, int cc, int M, int kk, uint32_t b0,
                                uint32_t above0, RtFinalLds &F, int32_t *io, float *so) {
  const int tid = (int)threadIdx.x;
  uint32_t k[P];
  int32_t pos[P];
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int i = tid + 256 * j;
    int a = 0;
#pragma unroll
    for (int step = kCandMaxChunks / 2; step > 0; step >>= 1) a = (int)F.soff[a + step] <= i ? a + step : a;
    const int sl = min(a * cc + (i - (int)F.soff[a]), kCandSlots - 1);
    const uint32_t kv = rk[sl];
    const int32_t pv = rp[sl];
    k[j] = i < M ? kv : 0u;
    pos[j] = i < M ? pv : 0;
  }
  // level 1: the next 11 bits of the keys in bin b0 (the bitmaps cleared alongside)
  RtThr t{b0, above0, (uint32_t)kk - above0};
  for (int i = tid; i < kRtBins; i += 256) F.lh[i] = 0u;
  for (int i = tid; i < 2 * kRtMapWords; i += 256) (&F.bm[0][0])[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (k[j] && (k[j] >> 21) == b0) atomicAdd(&F.lh[(k[j] >> 10) & 2047u], 1u);
  __syncthreads();
  t = rt_next(F.lh, kRtBins, 11, t, F.sh);
  // level 2: the last 10 bits of the keys under that 22-bit prefix
  for (int i = tid; i < 1024; i += 256) F.lh[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < P; ++j)
    if (k[j] && (k[j] >> 10) == t.prefix) atomicAdd(&F.lh[k[j] & 1023u], 1u);
  __syncthreads();
  t = rt_next(F.lh, 1024, 10, t, F.sh);
  const uint32_t tstar = t.prefix, quota = t.want;
  const uint32_t neq = F.lh[tstar & 1023u];   // every key equal to t* was counted in its level-2 bin
  const int nw = (M + 31) / 32;
  uint64_t pick = 0ull;
  if (neq > quota) {   // ties at t*: the equal keys lowest in position order
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = tid + 256 * j;
      if (k[j] == tstar) atomicOr(&F.bm[0][i >> 5], 1u << (i & 31));
    }
    __syncthreads();
    rt_word_prefix(F.bm[0], F.wpre, nw, F.sh);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int i = tid + 256 * j, w = i >> 5;
      if (k[j] == tstar && F.wpre[w] + __popc(F.bm[0][w] & ((1u << (i & 31)) - 1u)) < quota) pick |= 1ull << j;
    }
    __syncthreads();   // F.wpre is rewritten below
  } else {
#pragma unroll
    for (int j = 0; j < P; ++j) pick |= k[j] == tstar ? 1ull << j : 0ull;
  }
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int i = tid + 256 * j;
    if (k[j] > tstar) pick |= 1ull << j;
    if ((pick >> j) & 1ull) atomicOr(&F.bm[1][i >> 5], 1u << (i & 31));
  }
  __syncthreads();
  rt_word_prefix(F.bm[1], F.wpre, nw, F.sh);
#pragma unroll
  for (int j = 0; j < P; ++j)
    if ((pick >> j) & 1ull) {
      const int i = tid + 256 * j, w = i >> 5;
      const uint32_t slot = F.wpre[w] + __popc(F.bm[1][w] & ((1u << (i & 31)) - 1u));
      io[slot] = pos[j];
      if (so) so[slot] = keyf(k[j]);
    }
}

// The picks of long row r from its candidates (or from the whole row when a
// chunk's candidates overflowed), and the -1 tail.  Block-wide.

__device__ __forceinline__ void rt_final_row(int r, int n, int kk, const float *scores, int64_t ld, int topk, int nch, int cc,
                             const uint32_t *ckey, const int32_t *cpos, const uint32_t *cr, int32_t *idx_out,
                             float *score_out, RtFinalLds &F) {
  int32_t *io = idx_out + (int64_t)r * topk;
  float *so = score_out ? score_out + (int64_t)r * topk : nullptr;
  if (kk == n) {   // everything visible is taken, in order
    for (int j = threadIdx.x; j < n; j += 256) {
      io[j] = j;
      if (so) so[j] = scores[(int64_t)r * ld + j];
    }
  } else {
    // chunk counts -> exclusive offsets (wave 0), overflow flag
    if (threadIdx.x < 64) {
      const int c = threadIdx.x;
      const uint32_t v = c < nch ? cr[c] : 0u;
      uint32_t inc = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o, 64);
        if (c >= o) inc += t;
      }
      F.soff[c] = inc - v;
      if (c == 63) F.soff[kCandMaxChunks] = inc;
      const bool over = __ballot(v > (uint32_t)cc) != 0ull;
      if (c == 0) F.over = over ? 1 : 0;
    }
    __syncthreads();
    const int M = (int)F.soff[kCandMaxChunks];
    const uint32_t *rk = ckey + (int64_t)r * kCandSlots;
    const int32_t *rp = cpos + (int64_t)r * kCandSlots;
    const uint32_t b0 = cr[kCandMaxChunks], ab = cr[kCandMaxChunks + 1];
    // more than 8192 candidates (heavy ties at the edge): the whole-row select
    if (F.over || M > 256 * 32) rt_row_select(scores, ld, r, n, kk, io, so, F.lh, F.sh);
    else if (M <= 256 * 8) rt_cands_select<8>(rk, rp, nch, cc, M, kk, b0, ab, F, io, so);
    else if (M <= 256 * 16) rt_cands_select<16>(rk, rp, nch, cc, M, kk, b0, ab, F, io, so);
    else rt_cands_select<32>(rk, rp, nch, cc, M, kk, b0, ab, F, io, so);
  }
  for (int j = kk + (int)threadIdx.x; j < topk; j += 256) {
    io[j] = -1;
    if (so) so[j] = -INFINITY;
  }
}

// grid (T, nch), 256 threads: chunk c = positions [c*chunk, (c+1)*chunk) of
// row r.  Candidates (keys in the level-0 bins from b0 up) go to slots
// [c*cc, c*cc + cc) of the row's kCandSlots, in position order; the chunk's
// true candidate count goes to ccnt[r, c], and chunk 0 records b0 and the
// count of keys in the bins above it.
__global__ __launch_bounds__(256) void k_rt_cand(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                 const int32_t *__restrict__ count, int m,
                                                 const float *__restrict__ scores, int64_t ld, int topk,
                                                 const uint32_t *__restrict__ hist0, int chunk, int cc,
                                                 uint32_t *__restrict__ ckey, int32_t *__restrict__ cpos,
                                                 uint32_t *__restrict__ ccnt) {
  __shared__ uint32_t sh[8];
  const int r = blockIdx.x, c = blockIdx.y, nch = gridDim.y;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  const int kk = min(topk, n);
  const int lo = c * chunk, hi = min(n, lo + chunk);
  uint32_t total = 0, kmin_bin = 0, kmin_above = 0;
  if (kk < n && lo < n) {
    uint32_t k[16];
    rt_load(scores, ld, r, lo, hi, k);   // in flight during the histogram search
    uint32_t above;
    const int b0 = rt_find(hist0 + (int64_t)r * kRtBins, kRtBins, (uint32_t)kk, &above, sh);
    kmin_bin = (uint32_t)b0;
    kmin_above = above;
    const uint32_t kmin = (uint32_t)b0 << 21;
    uint32_t *ok = ckey + (int64_t)r * kCandSlots + (int64_t)c * cc;
    int32_t *op = cpos + (int64_t)r * kCandSlots + (int64_t)c * cc;
    for (int base = lo; base < hi; base += kRtChunk) {
      if (base != lo) rt_load(scores, ld, r, base, hi, k);
#pragma unroll
      for (int q = 0; q < 4; ++q) {   // position order: q, then thread, then e
        uint32_t ne = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) ne += k[4 * q + e] >= kmin ? 1u : 0u;
        uint32_t tot;
        uint32_t slot = total + tk_scan(ne, sh, &tot);
        total += tot;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (k[4 * q + e] < kmin) continue;
          if (slot < (uint32_t)cc) {
            ok[slot] = k[4 * q + e];
            op[slot] = base + 4 * ((int)threadIdx.x + 256 * q) + e;
          }
          ++slot;
        }
      }
    }
  }
  uint32_t *cr = ccnt + (int64_t)r * kCandRow;
  if (threadIdx.x == 0) {
    cr[c] = total;
    if (c == 0 && kk < n) {
      cr[kCandMaxChunks] = kmin_bin;
      cr[kCandMaxChunks + 1] = kmin_above;
    }
  }
}

// grid (T), 256 threads: the picks of each long row from its candidates
__global__ __launch_bounds__(256) void k_rt_final(const int32_t *__restrict__ seq, const int32_t *__restrict__ tok,
                                                  const int32_t *__restrict__ count, int m,
                                                  const float *__restrict__ scores, int64_t ld, int topk, int nch,
                                                  int cc, const uint32_t *__restrict__ ckey,
                                                  const int32_t *__restrict__ cpos, const uint32_t *__restrict__ ccnt,
                                                  int32_t *__restrict__ idx_out, float *__restrict__ score_out) {
  __shared__ RtFinalLds F;
  const int r = gridDim.x - 1 - blockIdx.x;
  const int n = n_visible(tok[r], m, count[seq[r]]);
  rt_final_row(r, n, min(topk, n), scores, ld, topk, nch, cc, ckey, cpos, ccnt + (int64_t)r * kCandRow, idx_out,
               score_out, F);
}

// Scratch memory of dsv4_index_topk_noalloc (the score rows, histograms,
// per-chunk counts and thresholds that dsv4_index_topk keeps in the caller's
// workspace).  One copy per GPU, held until the process ends; host code never
// passes this name to a kernel, only the address hipGetSymbolAddress returns.
constexpr size_t kNoAllocScratchBytes = DSV4_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

size_t index_topk_scratch_bytes() { return kNoAllocScratchBytes; }

// Device address of this GPU's scratch array, looked up once per device (with
// that device current) and kept for later calls.
int index_topk_scratch(void **ptr) {
  static std::mutex mu;
  static std::map<int, void *> addr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(DSV4_EHIP, "index_topk_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  auto it = addr.find(dev);
  if (it == addr.end()) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DSV4_EHIP, "index_topk_noalloc: scratch address on device %d: %s", dev, hipGetErrorString(e));
    it = addr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return DSV4_OK;
}

// Top-k plan: rows of at most 16384 entries are selected by one workgroup
// each (k_topk_chunk, KPT keys per thread); longer rows by the candidate
// path (level-0 histogram, k_rt_cand over at most kCandMaxChunks chunks of
// `chunk` entries with cc candidate slots each, then k_rt_final).  Workspace: the
// score rows, then (long rows) the histograms, the per-chunk candidate counts,
// the candidate keys and their positions.
struct TopkPlan {
  bool radix;
  int kpt, nch, chunk, cc;
  size_t scores_bytes, hist_bytes, cnt_bytes, cand_bytes;
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
  p.scores_bytes = align256((size_t)n_rows * (size_t)st * 4);
  if (p.radix) {
    int64_t nch = std::min<int64_t>(kCandMaxChunks, (st + kRtChunk - 1) / kRtChunk);
    const int64_t chunk = ((st + nch - 1) / nch + kRtChunk - 1) / kRtChunk * kRtChunk;
    nch = (st + chunk - 1) / chunk;
    p.nch = (int)nch;
    p.chunk = (int)chunk;
    p.cc = kCandSlots / p.nch;
    p.hist_bytes = align256((size_t)n_rows * kRtBins * 4);
    p.cnt_bytes = align256((size_t)n_rows * kCandRow * 4);
    p.cand_bytes = align256((size_t)n_rows * kCandSlots * 4);
  }
  (void)topk;
  return p;
}

size_t index_topk_ws(int64_t n_rows, int64_t stride, int topk) {
  const TopkPlan p = plan_topk(n_rows, stride, topk);
  return p.scores_bytes + p.hist_bytes + p.cnt_bytes + 2 * p.cand_bytes + 256;
}

int index_topk_supported(int64_t stride, int topk) {
  // grid.y holds a row's chunks: 1024-entry chunks of the fp32 scoring kernel
  // (the most of any pass: the radix passes take 4096, the MFMA scans at least
  // 31 * 128 entries per workgroup)
  return (stride + 1023) / 1024 <= 65535 && topk >= 1;
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
  uint32_t *hist0 = p.radix ? (uint32_t *)((char *)ws + p.scores_bytes) : nullptr;
  uint32_t *ccnt = p.radix ? (uint32_t *)((char *)hist0 + p.hist_bytes) : nullptr;
  uint32_t *ckey = p.radix ? (uint32_t *)((char *)ccnt + p.cnt_bytes) : nullptr;
  int32_t *cpos = p.radix ? (int32_t *)((char *)ckey + p.cand_bytes) : nullptr;
  if (p.radix) {   // the level-0 histograms start at zero (a kernel, so graphs may capture it)
    const int64_t hw = (int64_t)T * kRtBins;
    hipLaunchKernelGGL(k_rt_zero, dim3((unsigned)((hw + 255) / 256)), dim3(256), 0, st, hist0, hw);
  }
  bool hist_built = false;   // the decode scoring kernel builds the level-0 histograms
  IdxQ Q{q->seq, q->tok, qv, qscale, w, H, Di};
  IdxK K{kp->data, kp->blk_scale, kp->count, kp->seq_stride, m};
  const int64_t ld = kp->seq_stride;
  // scoring kernels with one workgroup per (query row, entry chunk)
  typedef void (*ScoreK)(IdxQ, IdxK, float, uint32_t *, float *, int64_t);
  ScoreK sk = nullptr;
  int eb = 1;   // entries per wave iteration / 16
  if (q_dtype == DSV4_MXFP4) {
    eb = 1;   // one 16-entry block per wave iteration (measured against 2, 4 and 8: 34.3 -> 32.2 us, 1M decode)
    switch (H / 16) {
    case 1: sk = k_index_scores_mfma<1, 1, true, 1>; break;
    case 2: sk = k_index_scores_mfma<2, 1, true, 1>; break;
    case 3: sk = k_index_scores_mfma<3, 1, true, 1>; break;
    default: sk = k_index_scores_mfma<4, 1, true, 1>; break;
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
    // two thirds of what is resident at once: swept at 1/2, 2/3 and all of it,
    // the CSA decode scan took 60.8, 51.7 and 54.3 us, the MXFP4 scan of the 1M
    // mixed decode 33.0, 32.1 and 33.4 us (fewer concurrent streams per CU; both
    // rows' super-blocks then also divide evenly over their workgroups)
    int64_t per_row = std::min<int64_t>(std::max<int64_t>(1, 2 * resident_wgs((const void *)sk, 256) / 3 / T),
                                        std::max<int64_t>(1, blocks));
    // at most kScoreStage / unit - 1 super-blocks per workgroup (its LDS staging)
    const int64_t cap = kScoreStage / unit - 1;
    per_row = std::max<int64_t>(per_row, (blocks + cap - 1) / cap);
    hipLaunchKernelGGL(sk, dim3(T, (unsigned)per_row), dim3(256), 0, st, Q, K, scale, hist0, scores, ld);
    hist_built = hist0 != nullptr;
  } else {
    constexpr int QPW = 1;   // queries per wave (4 per workgroup share each key tile)
    dim3 g8((T + 4 * QPW - 1) / (4 * QPW));
    // rows whose picks are all their visible entries need no score unless the
    // pick scores are returned (k_topk_chunk reads them only then; the long-row
    // path reads every row's scores)
    const int skip_n = (!p.radix && !score_out) ? topk : 0;
    switch (H / 16) {
    case 1: hipLaunchKernelGGL((k_index_scores_q8<1, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, skip_n, scores, ld); break;
    case 2: hipLaunchKernelGGL((k_index_scores_q8<2, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, skip_n, scores, ld); break;
    case 3: hipLaunchKernelGGL((k_index_scores_q8<3, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, skip_n, scores, ld); break;
    default: hipLaunchKernelGGL((k_index_scores_q8<4, QPW>), g8, dim3(256), 0, st, Q, K, scale, T, skip_n, scores, ld); break;
    }
  }
  int rc = check_launch("k_index_scores");
  if (rc) return rc;
  if (!p.radix) {
#define DSV4_TK1(KPT, NT)                                                                                        \
  hipLaunchKernelGGL((k_topk_chunk<KPT, NT>), dim3(T), dim3(NT), 0, st, q->seq, q->tok, kp->count, m, scores, ld, \
                     topk, idx_out, score_out)
    // rows of up to 2048 entries on 128 threads (twice the keys per thread):
    // at S = 8192 the select took 41.3 us on 256 threads, 37.4 on 128, 38.6 on 64
    switch (p.kpt) {
    case 4: DSV4_TK1(8, 128); break;
    case 8: DSV4_TK1(16, 128); break;
    case 16: DSV4_TK1(16, 256); break;
    case 32: DSV4_TK1(32, 256); break;
    default: DSV4_TK1(64, 256); break;
    }
#undef DSV4_TK1
    return check_launch("k_topk_chunk");
  }
  if (!hist_built) {
    const dim3 g((unsigned)T, (unsigned)((kp->seq_stride + kRtChunk - 1) / kRtChunk));
    hipLaunchKernelGGL(k_rt_hist0, g, dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld, topk, hist0);
  }
  hipLaunchKernelGGL(k_rt_cand, dim3((unsigned)T, (unsigned)p.nch), dim3(256), 0, st, q->seq, q->tok, kp->count, m,
                     scores, ld, topk, hist0, p.chunk, p.cc, ckey, cpos, ccnt);
  hipLaunchKernelGGL(k_rt_final, dim3((unsigned)T), dim3(256), 0, st, q->seq, q->tok, kp->count, m, scores, ld,
                     topk, p.nch, p.cc, ckey, cpos, ccnt, idx_out, score_out);
  return check_launch("k_rt_final");
}

}  // namespace dsv4host
