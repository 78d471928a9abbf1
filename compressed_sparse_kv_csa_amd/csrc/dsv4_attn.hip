// dsv4_attn.hip -- CSA / HCA core attention with one shared K=V head, for gfx950.
//
// HF DeepSeek-V4 page, "Hybrid attention" backbone: multi-query attention with a
// single K=V head read as both key and value; partial RoPE on the last
// qk_rope_head_dim channels with the inverse rotation (-p) on the output slice;
// a learned per-head sink; a sliding-window K=V branch concatenated with the
// compressor's entries.  "Attention mask layout": CSA queries see the
// indexer's picks (-1 masked), HCA queries every entry w < (t+1)/m.
//
// Per query row r (sequence b, token t, position p) the row list is
//   [window rows holding tokens max(t-W+1, first_tok) .. t] ++ [pool rows]
// (CSA: the valid idx[r, :], HCA: entries 0 .. min(count, (t+1)/m) - 1).
//
// k_attn_mfma<D, NW, FP8>: one workgroup per (query row, row split).  The 64
// query heads are the MFMA dimension that is shared by every row (MQA), so a
// 32-row K=V tile is staged once in LDS and used by all heads:
//   Ks [32][D+8]  row-major  -> A operand of S^T = K q~^T   (16x16x32 f16)
//   Vt [D][32+4]  transposed -> A operand of O^T = V^T P^T  (16x16x32 f16)
// Wave w owns heads 16w..16w+15: q~ (rotated, scaled by sm_scale*log2 e) stays
// in registers as the B operand, the 16x16 score tile S^T lands with each lane
// holding 8 rows of one head, which is exactly the B-operand layout P^T needs
// for the PV product (no shuffle of P), and O^T accumulates with each lane
// holding 4 dims of the same head (so the online-softmax rescale is per lane).
// The tile, q~ and P are fp16 on the matrix cores: a stored bf16 value whose
// magnitude lies in [2^-14, 65504] is exact in fp16 (smaller ones lose
// significand bits to fp16's subnormals, larger ones overflow; the callers'
// rows and queries are far inside that range), and fp16's 11-bit significand
// keeps the rounding of q~ and P four times smaller than bf16 would, which
// matters when a query has only a few rows and every logit error moves the
// output directly.  FP8 rows
// (E4M3 x row scale, bf16 rope channels) are decoded to fp16 while staging.
// Several splits per query (decode) each write their output normalised by
// their own sum (fp16: a convex combination of rows stays in the rows' range)
// with their (max, sum) in fp32; k_attn_combine merges them with the sink.
//
// k_attn_f32: scalar fp32 path for small fp32 shapes.
#include "dsv4_common.h"

#include <atomic>
#include <type_traits>

namespace dsv4 {

struct RowSrc {
  const uint8_t *data;
  const float *rscale;
  const int32_t *count;
  const int32_t *first_tok;
  int64_t stride;
  int64_t rbytes;
  int dtype, tail;
  int ring;   // windows: token j at row j mod stride
};

struct AttnArgs {
  const int32_t *seq, *tok;
  const int64_t *pos0;
  const void *q;
  int T, H, qdtype;
  RowSrc win;
  int W;
  RowSrc pool;
  const int32_t *idx;
  int topk, m, csa;
  const float *sinks;
  float scale_log2;   // sm_scale * log2(e)
  int rope_dim;
  double theta;
  double inv_freq[32];   // theta^(-2i/rope_dim), fp64, filled on the host
  void *out;
  int out_dtype;
  int nsplit;
  uint16_t *part_o;   // [T*nsplit*H, D] fp16: each split's output normalised by its own sum
  float *part_ml;     // [T*nsplit*H, 2]: the split's reference maximum (log2 units) and sum
  int diag;           // count into g_diag (dsv4_set_diagnostics)
};

// Diagnostic counters of this GPU (DSV4_DIAG_*), added to only while
// dsv4_set_diagnostics is on: raises of the fixed softmax reference inside a
// tile, and pick entries that are neither -1 nor below the pool count.
__device__ unsigned long long g_diag[DSV4_DIAG_COUNT];

constexpr int kMaxSel = 2048;

// Rows of one query: window part [0, nwin) then pool part.
struct RowPlan {
  int b, t, nwin, nsel, wlo;
  int pcount;   // the sequence's pool entries (0 without a pool)
  int64_t p;
};

// read in place of absent per-sequence arrays (never written)
__device__ int32_t kZeroI32[1];
__device__ int64_t kZeroI64[1];

// The plan's loads go out in two rounds: the row's (sequence, token), then the
// sequence's pos0, window first token and count, and pool count.  An absent
// array reads a zero stand-in, so that no load waits behind a branch on an
// argument (each such branch cost a scalar round trip).
__device__ __forceinline__ RowPlan row_plan(const AttnArgs &A, int r) {
  const int b = A.seq[r];
  const int t = A.tok[r];
  const bool win = A.W > 0, pool = A.pool.data != nullptr;
  const int64_t p0 = *(A.pos0 ? A.pos0 + b : kZeroI64);
  const int ft = *(win && A.win.first_tok ? A.win.first_tok + b : kZeroI32);
  const int wc = *(win ? A.win.count + b : kZeroI32);
  const int pc = *(pool ? A.pool.count + b : kZeroI32);
  // every value needed here: the compiler would otherwise sink each load into
  // the branch that uses it, one round trip after another (r is uniform, so
  // are they)
  asm volatile("" ::"s"(t), "s"(p0), "s"(ft), "s"(wc), "s"(pc));
  RowPlan P;
  P.b = b;
  P.t = t;
  P.p = p0 + t;
  P.pcount = pc;
  P.nwin = 0;
  P.wlo = 0;
  if (win) {
    const int lo = max(max(t - A.W + 1, ft), 0);
    const int hi = min(t, ft + wc - 1);
    // storage row of the first window token; the rows of the later ones
    // follow it, wrapping at the stride (only a ring ever wraps)
    P.wlo = A.win.ring ? (int)(lo % A.win.stride) : lo - ft;
    P.nwin = hi >= lo ? hi - lo + 1 : 0;
  }
  P.nsel = !A.csa && pool ? min((t + 1) / A.m, pc) : 0;
  return P;
}

// Compact the valid entries of idx[r, :] (>= 0 and < count) into sel[],
// preserving order.  Block-wide; every index load is issued before the one
// barrier; returns the count (sel[] is visible after the caller's next
// barrier).  sh_cnt holds kMaxSel/64 ints.
// The index entries of query row r a workgroup of NT threads compacts:
// thread t holds entries t, t + NT, ... (issued early, used by compact_idx).
template <int NT>
struct IdxPre {
  int v[kMaxSel / NT];
};
template <int NT>
__device__ __forceinline__ IdxPre<NT> load_idx(const AttnArgs &A, int r) {
  constexpr int PER = kMaxSel / NT;
  IdxPre<NT> p;
  const int nq = (A.topk + NT - 1) / NT;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = q * NT + (int)threadIdx.x;
    p.v[q] = (q < nq && i < A.topk) ? A.idx[(int64_t)r * A.topk + i] : -1;
  }
  return p;
}

// Compact the valid entries of idx[r, :] (>= 0 and < count) into sel[],
// preserving order.  Block-wide, one barrier; returns the count (sel[] is
// visible after the caller's next barrier).  sh_cnt holds kMaxSel/64 ints.
template <int NT>
__device__ int compact_idx(const AttnArgs &A, const IdxPre<NT> &pre, int cnt, int *sel, int *sh_cnt,
                           bool count_bad = false) {
  constexpr int NWV = NT / 64, PER = kMaxSel / NT;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nq = (A.topk + NT - 1) / NT;
  if (A.diag && count_bad) {   // entries past the row's end load as -1
    unsigned long long nb = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) nb += (q < nq && pre.v[q] != -1 && !(pre.v[q] >= 0 && pre.v[q] < cnt)) ? 1ull : 0ull;
    if (nb) atomicAdd(&g_diag[DSV4_DIAG_BAD_PICKS], nb);
  }
  unsigned long long bal[PER];
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    bal[q] = __ballot(pre.v[q] >= 0 && pre.v[q] < cnt);
    if (lane == 0 && q < nq) sh_cnt[q * NWV + wv] = __popcll(bal[q]);
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    if (q >= nq) break;
    int off = total;
    for (int w = 0; w < NWV; ++w) {
      const int cw = sh_cnt[q * NWV + w];
      off += w < wv ? cw : 0;
      total += cw;
    }
    if ((bal[q] >> lane) & 1ull) sel[off + __popcll(bal[q] & ((1ull << lane) - 1ull))] = pre.v[q];
  }
  return total;
}
template <int NT>
__device__ int compact_idx(const AttnArgs &A, int r, int cnt, int *sel, int *sh_cnt, bool count_bad = false) {
  return compact_idx<NT>(A, load_idx<NT>(A, r), cnt, sel, sh_cnt, count_bad);
}

// storage row (within its sequence) of window row i of a query
__device__ __forceinline__ int win_slot(const AttnArgs &A, const RowPlan &P, int i) {
  const int s = P.wlo + i;
  return s >= A.win.stride ? s - (int)A.win.stride : s;
}

__device__ __forceinline__ const uint8_t *row_ptr(const AttnArgs &A, const RowPlan &P, const int *sel, int i,
                                                  float *scale) {
  if (i < P.nwin) {
    const int64_t g = (int64_t)P.b * A.win.stride + win_slot(A, P, i);
    *scale = A.win.rscale ? A.win.rscale[g] : 1.f;
    return A.win.data + g * A.win.rbytes;
  }
  const int s = A.csa ? sel[i - P.nwin] : i - P.nwin;
  const int64_t g = (int64_t)P.b * A.pool.stride + s;
  *scale = A.pool.rscale ? A.pool.rscale[g] : 1.f;
  return A.pool.data + g * A.pool.rbytes;
}

__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  return pack_f16x2(bf16_to_f32((uint16_t)(v & 0xFFFFu)), bf16_to_f32((uint16_t)(v >> 16)));
}

// 8 channels [8*c8, 8*c8+8) of a stored row -> 8 fp16 (packed in a u32x4)
template <int D, bool FP8>
__device__ __forceinline__ u32x4 load8(const uint8_t *row, int c8, float scale, int tail) {
  const int d0 = 8 * c8;
  if (!FP8 || d0 >= D - tail) {
    const u32x4 v = FP8 ? *reinterpret_cast<const u32x4 *>(row + (D - tail) + 2 * (d0 - (D - tail)))
                        : *reinterpret_cast<const u32x4 *>(row + 16 * c8);
    return u32x4{bf16x2_to_f16x2(v.x), bf16x2_to_f16x2(v.y), bf16x2_to_f16x2(v.z), bf16x2_to_f16x2(v.w)};
  }
  const u32x2 v = *reinterpret_cast<const u32x2 *>(row + d0);
  u32x4 o;
  o.x = pack_f16x2(e4m3_to_f32(v.x & 255u) * scale, e4m3_to_f32((v.x >> 8) & 255u) * scale);
  o.y = pack_f16x2(e4m3_to_f32((v.x >> 16) & 255u) * scale, e4m3_to_f32(v.x >> 24) * scale);
  o.z = pack_f16x2(e4m3_to_f32(v.y & 255u) * scale, e4m3_to_f32((v.y >> 8) & 255u) * scale);
  o.w = pack_f16x2(e4m3_to_f32((v.y >> 16) & 255u) * scale, e4m3_to_f32(v.y >> 24) * scale);
  return o;
}

template <int D, int NW, bool FP8>
__global__ __launch_bounds__(NW * 64) void k_attn_mfma(AttnArgs A) {
  constexpr int NT = NW * 64;
  constexpr int KP = D + 8;   // Ks row pitch (fp16 elements)
  constexpr int VP = 36;      // Vt row pitch (fp16 elements)
  constexpr int NJ = D / 32;  // k-steps of the QK product
  constexpr int NDB = D / 16; // 16-dim blocks of the output
  __shared__ __attribute__((aligned(16))) uint16_t Ks[32 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];
  __shared__ int sel[kMaxSel];
  __shared__ float rc[32], rs[32];
  __shared__ int sh_cnt[kMaxSel / 64];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int r = (A.T - 1) - (int)(blockIdx.x / A.nsplit);   // longest rows first
  const int split = blockIdx.x % A.nsplit;
  // raw bf16 query loads first: their latency hides behind the setup below
  const int h = 16 * wv + c;
  f16x8 qb[NJ];
  {
    const uint16_t *qr = (const uint16_t *)A.q + ((int64_t)r * A.H + h) * D + 8 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) qb[j] = *reinterpret_cast<const f16x8 *>(qr + 32 * j);
  }
  RowPlan P = row_plan(A, r);
  if (A.csa && A.topk > 0) P.nsel = compact_idx<NT>(A, r, P.pcount, sel, sh_cnt, blockIdx.x % A.nsplit == 0);
  const int nrows = P.nwin + P.nsel;
  const int ntiles = (nrows + 31) / 32;
  const int tps = (ntiles + A.nsplit - 1) / A.nsplit;
  const int tile_lo = split * tps;
  const int tile_hi = min(ntiles, tile_lo + tps);
  const int R = A.rope_dim;

  if (tid < R / 2) rope_cs_f((double)P.p, A.inv_freq[tid], 1.f, &rc[tid], &rs[tid]);
  __syncthreads();

  // q~ = RoPE(q) * sm_scale * log2(e) as the B operand: lane holds head h,
  // dims 32j + 8g .. +8
  {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d0 = 32 * j + 8 * g;
      u32x4 raw;
      __builtin_memcpy(&raw, &qb[j], 16);
      float x[8];
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_to_f32((uint16_t)(wds[k] & 0xFFFF));
        x[2 * k + 1] = bf16_to_f32((uint16_t)(wds[k] >> 16));
      }
      if (d0 >= D - R) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pi = (d0 + 2 * k - (D - R)) >> 1;
          const float cs = rc[pi], sn = rs[pi];
          const float a = x[2 * k] * cs - x[2 * k + 1] * sn, bb = x[2 * k] * sn + x[2 * k + 1] * cs;
          x[2 * k] = a;
          x[2 * k + 1] = bb;
        }
      }
      u32x4 o;
      o.x = pack_f16x2(x[0] * A.scale_log2, x[1] * A.scale_log2);
      o.y = pack_f16x2(x[2] * A.scale_log2, x[3] * A.scale_log2);
      o.z = pack_f16x2(x[4] * A.scale_log2, x[5] * A.scale_log2);
      o.w = pack_f16x2(x[6] * A.scale_log2, x[7] * A.scale_log2);
      __builtin_memcpy(&qb[j], &o, 16);
    }
  }

  f32x4 acc_o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc_o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int tile = tile_lo; tile < tile_hi; ++tile) {
    const int base = tile * 32;
    __syncthreads();   // previous tile fully consumed
    // stage 32 rows: item = (row quad q4, 8-channel chunk c8)
    for (int it = tid; it < 8 * (D / 8); it += NT) {
      const int q4 = it / (D / 8), c8 = it % (D / 8);
      u32x4 v[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int i = base + 4 * q4 + rr;
        if (i < nrows) {
          float sc;
          const uint8_t *rp = row_ptr(A, P, sel, i, &sc);
          v[rr] = load8<D, FP8>(rp, c8, sc, i < P.nwin ? A.win.tail : A.pool.tail);
        } else {
          v[rr] = u32x4{0u, 0u, 0u, 0u};
        }
        *reinterpret_cast<u32x4 *>(&Ks[(4 * q4 + rr) * KP + 8 * c8]) = v[rr];
      }
      // transpose into Vt[dim][row]: 4 rows of one dim are 8 contiguous bytes
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t a0 = v[0][k], a1 = v[1][k], a2 = v[2][k], a3 = v[3][k];
        const u32x2 lo2 = u32x2{(a0 & 0xFFFFu) | (a1 << 16), (a2 & 0xFFFFu) | (a3 << 16)};
        const u32x2 hi2 = u32x2{(a0 >> 16) | (a1 & 0xFFFF0000u), (a2 >> 16) | (a3 & 0xFFFF0000u)};
        *reinterpret_cast<u32x2 *>(&Vt[(8 * c8 + 2 * k) * VP + 4 * q4]) = lo2;
        *reinterpret_cast<u32x2 *>(&Vt[(8 * c8 + 2 * k + 1) * VP + 4 * q4]) = hi2;
      }
    }
    __syncthreads();

    // S^T (rows x heads) = K q~^T : two 16-row blocks
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const uint16_t *kr = &Ks[(16 * mb + c) * KP + 8 * g];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const f16x8 a = *reinterpret_cast<const f16x8 *>(kr + 32 * j);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, qb[j], acc, 0, 0, 0);
      }
      s[mb] = acc;
    }
    // lane holds head h, rows base + 16mb + 4g + i
    float mloc = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = base + 16 * mb + 4 * g + i;
        if (row >= nrows) s[mb][i] = -INFINITY;
        mloc = fmaxf(mloc, s[mb][i]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);   // finite: every tile has a valid row
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f, p[8];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[4 * mb + i] = exp2f(s[mb][i] - m_new);
        psum += p[4 * mb + i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    u32x4 pw;
    pw.x = pack_f16x2(p[0], p[1]);
    pw.y = pack_f16x2(p[2], p[3]);
    pw.z = pack_f16x2(p[4], p[5]);
    pw.w = pack_f16x2(p[6], p[7]);
    f16x8 pb;
    __builtin_memcpy(&pb, &pw, 16);
    // O^T (dims x heads) += V^T P^T ; k index 8g+i <-> tile row 4g+i (i<4), 16+4g+(i-4)
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const uint16_t *vr = &Vt[(16 * db + c) * VP];
      const u32x2 lo = *reinterpret_cast<const u32x2 *>(vr + 4 * g);
      const u32x2 hi = *reinterpret_cast<const u32x2 *>(vr + 16 + 4 * g);
      const u32x4 av = u32x4{lo.x, lo.y, hi.x, hi.y};
      f16x8 a;
      __builtin_memcpy(&a, &av, 16);
      f32x4 o = acc_o[db];
      o[0] *= alpha; o[1] *= alpha; o[2] *= alpha; o[3] *= alpha;
      acc_o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, o, 0, 0, 0);
    }
  }

  // row sums of the four lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);

  if (A.nsplit > 1) {
    const int64_t pr = ((int64_t)r * A.nsplit + split) * A.H + h;
    uint16_t *po = A.part_o + pr * D;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;   // normalised: within the rows' range, fp16-safe
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const f32x4 a = acc_o[db];
      *reinterpret_cast<u32x2 *>(po + 16 * db + 4 * g) =
          u32x2{pack_f16x2(a[0] * inv, a[1] * inv), pack_f16x2(a[2] * inv, a[3] * inv)};
    }
    if (g == 0) {
      A.part_ml[2 * pr] = m_run;
      A.part_ml[2 * pr + 1] = l_run;
    }
    return;
  }

  float f = 1.f, den = l_run;
  if (A.sinks) {
    const float sg = A.sinks[h] * kLog2e;
    const float M = fmaxf(m_run, sg);
    f = exp2f(m_run - M);
    den = l_run * f + exp2f(sg - M);
  }
  const float inv = den > 0.f ? f / den : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    float o[4];
    const int d0 = 16 * db + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = acc_o[db][i] * inv;
    if (d0 >= D - R) {
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int pi = (d0 + 2 * k - (D - R)) >> 1;
        const float cs = rc[pi], sn = rs[pi];
        const float a = o[2 * k] * cs + o[2 * k + 1] * sn, bb = -o[2 * k] * sn + o[2 * k + 1] * cs;
        o[2 * k] = a;
        o[2 * k + 1] = bb;
      }
    }
    const int64_t oe = ((int64_t)r * A.H + h) * D + d0;
    if (A.out_dtype == DSV4_F32) {
      *reinterpret_cast<f32x4 *>((float *)A.out + oe) = f32x4{o[0], o[1], o[2], o[3]};
    } else {
      *reinterpret_cast<u32x2 *>((uint16_t *)A.out + oe) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
  }
}

// ---------------------------------------------------------------- fp16 / FP8 rows, DMA-staged
// k_attn_f16<NHB, NW, FP8>: the fast path.  NW waves; for S^T each wave owns
// 16*NHB heads.  Rows are gathered straight from global memory into LDS with
// global_load_lds_dwordx4 (no VGPR staging), double-buffered: the gather of
// tile i+1 is in flight while tile i is on the matrix cores.  The PV operand
// V^T comes from the same row-major fp16 tile through ds_read_b64_tr_b16 (a
// 16x4 transpose inside each 16-lane group), so no transposed copy is written.
//
// fp16 rows with 16, 32 or 64 heads split PV by output channel instead of by
// head: after S^T and the softmax, every wave writes its 16-head P^T fragment
// to LDS, and after one barrier wave w accumulates O^T for all heads over the
// 16-channel blocks w, w + NW, w + 2 NW, ... (a D/NW share, with the rotated
// last channels spread over all waves).  Each V^T fragment read from LDS then feeds
// NW matrix products, and the tile's V^T is read once per workgroup instead of
// once per wave (the transposing reads run at about half the rate of plain
// 16-byte reads).  The accumulators stay 128 VGPRs per wave either way.  The
// next tile's eight 1 KB row DMAs per wave are issued right before that
// barrier, where a wave waits for the others' scores anyway; a lane holds one
// row address so that each DMA is two lane reads and scalar LDS addressing.
// bf16 outputs are staged in the idle tile buffers, heads as rows, so that
// every global store writes a whole 1 KB head row.
//
// fp16 rows (prefill: the compressor and the rope kernel emit fp16) land in
// the tile as they are, one 1 KB row per wave instruction.  FP8 rows (decode
// caches: 448 E4M3 bytes x row scale, then 64 bf16 rope channels, 576 B) land
// as raw bytes, with their scales, in a raw buffer whose gather for tile i+1
// is spread over the QK^T steps of tile i; one block-wide pass then decodes
// the raw tile into the fp16 tile (scaled E4M3 -> fp16 conversion by the
// scale's power of two, exact, then one fp16 multiply by its significand;
// bf16 rope channels converted), so decoding is paid once per row per
// workgroup instead of once per wave and MFMA operand.
//
// Waits written out, not left to the compiler's tracking of LDS DMA:
// vm_wait_all: this wave's vector memory operations (DMAs included) are done.
// lds_barrier: LDS writes visible to the workgroup, outstanding DMAs kept in
// flight; the empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void vm_wait_all() { __builtin_amdgcn_s_waitcnt(0x0f70); }   // vmcnt(0)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) uint16_t lds_u16;

// a pointer every lane holds the same value of, in scalar registers
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T *)(((uint64_t)hi << 32) | lo);
}

constexpr float kRefSlack = 15.f;   // log2 units: P <= 2^15 stays finite in fp16

// FP8 rows: 448 E4M3 channels, then 64 bf16 channels
constexpr int kF8Nope = 448, kF8Row = kF8Nope + 2 * 64;
constexpr int kF8Chunks = 32 * kF8Row / 1024;   // 1 KB DMA instructions per 32-row raw tile

// R64: the rope width is the 64 channels of every configuration in the pages,
// fixed at compile time so that the per-block rotation tests fold away
template <int NHB, int NW, bool FP8, bool R64>
__global__ __launch_bounds__(NW * 64, FP8 ? 1 : 2) void k_attn_f16(AttnArgs A) {
  constexpr int D = 512, KP = D + 16, NJ = D / 32, NDB = D / 16, NT = NW * 64;
  constexpr int RB = FP8 ? kF8Row : 2 * D;   // stored row bytes
  // Dimension-split PV (fp16 rows, one 16-head block per wave, NW | 32): every
  // wave publishes its P^T fragment in LDS and accumulates O^T for all heads
  // over its own D/NW output channels, so each V^T fragment read from LDS feeds
  // NW products instead of one (the tile's V^T is read once per workgroup, not
  // once per wave).  AH: head blocks and DB: 16-channel blocks a wave accumulates.
  constexpr bool DSPV = NHB == 1 && (NW == 1 || NW == 2 || NW == 4);
  constexpr int AH = DSPV ? NW : NHB, DB = DSPV ? NDB / NW : NDB;
  // dimension-split PV: wave w owns the 16-channel blocks w, w + NW, w + 2 NW, ...
  // (so the rotated last channels are spread over all waves)
  constexpr int CS = DSPV ? NW : 1;
  static_assert(!FP8 || 32 * kF8Row % 1024 == 0, "raw tile must be whole DMA instructions");
  __shared__ __attribute__((aligned(16))) uint16_t T0[32 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t T1[FP8 ? 8 : 32 * KP];   // FP8 rows: one fp16 tile
  __shared__ __attribute__((aligned(16))) uint8_t RW[FP8 ? 32 * kF8Row : 16];
  __shared__ float RSC[FP8 ? 32 : 1];
  __shared__ int sel[kMaxSel];
  __shared__ float rc[32], rs[32];
  __shared__ float sk[64];   // the heads' sinks (log2 units), loaded with the setup
  __shared__ int sh_cnt[kMaxSel / 64];
  __shared__ uint32_t rfl;   // DSPV: byte w = wave w raised its heads' reference in this tile
  __shared__ float fsh[DSPV ? 64 : 1];   // the raise factors of those heads
  __shared__ __attribute__((aligned(16))) uint16_t PB[DSPV ? NW * 64 * 8 : 8];   // P^T fragments, wave-major

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int r = (A.T - 1) - (int)(blockIdx.x / A.nsplit);
  const int split = blockIdx.x % A.nsplit;
  // raw bf16 query loads first: their latency hides behind the setup below
  const int h0 = wv * 16 * NHB;
  f16x8 qb[NHB][NJ];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const uint16_t *qr = (const uint16_t *)A.q + ((int64_t)r * A.H + h0 + 16 * hb + c) * D + 8 * g;
#pragma unroll
    for (int j = 0; j < NJ; ++j) qb[hb][j] = *reinterpret_cast<const f16x8 *>(qr + 32 * j);
  }
  // the index entries next: their latency hides behind the row plan
  IdxPre<NT> ipre;
  if (A.csa && A.topk > 0) ipre = load_idx<NT>(A, r);
  RowPlan P = row_plan(A, r);
  const int R = R64 ? 64 : A.rope_dim;
  const int nwin = P.nwin, csa = A.csa;
  // row addressing in scalars: window rows first, then pool rows
  const uint8_t *pbase = A.pool.data ? A.pool.data + (int64_t)P.b * A.pool.stride * RB : nullptr;
  const uint8_t *wbase = A.win.data ? A.win.data + (int64_t)P.b * A.win.stride * RB : pbase;
  const float *psc = FP8 && A.pool.data ? A.pool.rscale + (int64_t)P.b * A.pool.stride : nullptr;
  const float *wsc = FP8 && A.win.data ? A.win.rscale + (int64_t)P.b * A.win.stride : psc;

  // Row ids: window storage row (>= 0) or -1 - pool entry.  Positions past the end of
  // the list are clamped to its last row, so every gathered tile row holds
  // finite stored values (their probabilities are zero) and no buffer needs
  // clearing.  nrows is provisional (window + HCA rows) until CSA compaction.
  int nrows = nwin + P.nsel;
  auto row_id = [&](int i) -> int {
    i = min(i, nrows - 1);
    return i < nwin ? win_slot(A, P, i) : -1 - (csa ? sel[i - nwin] : i - nwin);
  };
  constexpr int RPW = (32 + NW - 1) / NW;   // tile rows per wave (wave w: rows w, w+NW, ...)
  // lane k < RPW: global address of row wv + NW*k of the tile (0: no such row),
  // so that one DMA takes two lane reads and scalar LDS addressing
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  auto tile_addr = [&](int tile) -> uint64_t {
    if (!(lane < RPW && wv + NW * lane < 32)) return 0;
    const int rk = row_id(32 * tile + wv + NW * lane);
    return (uint64_t)(rk >= 0 ? wbase + (int64_t)rk * RB : pbase + (int64_t)(-1 - rk) * RB);
  };
  // when NW divides 32 every lane k < RPW holds a row address (positions past
  // the list are clamped to its last row), so no DMA is conditional
  const uint32_t loff = 16u * (uint32_t)lane;
  auto dma_row = [&](uint64_t ad, int k, uint16_t *T) {   // row wv + NW*k of a tile, one 1 KB DMA
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)ad, k);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(ad >> 32), k);
    const uint8_t *rp = (const uint8_t *)(((uint64_t)hi << 32) | lo);
    if (32 % NW == 0 || rp)
      __builtin_amdgcn_global_load_lds(rp + loff, (lds_void *)(lds_u16 *)(T + (wvs + NW * k) * KP), 16, 0, 0);
  };
  auto gather = [&](int tile, uint16_t *T) {
    const uint64_t ad = tile_addr(tile);
#pragma unroll
    for (int k = 0; k < RPW; ++k) dma_row(ad, k, T);
  };
  // the first tile can be in flight during the compaction when its rows are
  // known without it: window rows (CSA prefill: the newest 32 tokens) or HCA rows
  const bool early = !FP8 && A.nsplit == 1 && (csa ? nwin >= 32 : nrows > 0);
  if (early) gather(0, T0);
  if (csa && A.topk > 0) {
    P.nsel = compact_idx<NT>(A, ipre, P.pcount, sel, sh_cnt, split == 0);
    nrows = nwin + P.nsel;
  }
  const int ntiles = (nrows + 31) / 32;
  const int tps = (ntiles + A.nsplit - 1) / A.nsplit;
  const int tile_lo = split * tps;
  const int tile_hi = min(ntiles, tile_lo + tps);

  if (tid < R / 2) rope_cs_f((double)P.p, A.inv_freq[tid], 1.f, &rc[tid], &rs[tid]);
  if (tid < A.H) sk[tid] = A.sinks ? A.sinks[tid] * kLog2e : -INFINITY;
  __syncthreads();
  // the epilogue's output row and mode, formed now and held in scalars so that
  // the epilogue does not wait for argument reloads
  int e_ns = __builtin_amdgcn_readfirstlane(A.nsplit), e_odt = __builtin_amdgcn_readfirstlane(A.out_dtype);
  int e_H = __builtin_amdgcn_readfirstlane(A.H), e_sk = __builtin_amdgcn_readfirstlane(A.sinks != nullptr ? 1 : 0);
  uint16_t *orow = uniform_ptr((uint16_t *)A.out + (int64_t)r * A.H * D);
  uint16_t *e_po = uniform_ptr(A.part_o);
  float *e_pml = uniform_ptr(A.part_ml);
  asm volatile("" : "+s"(e_ns), "+s"(e_odt), "+s"(e_H), "+s"(e_sk));
  const bool stage = DSPV && !FP8 && e_ns == 1 && e_odt != DSV4_F32;

  // FP8: the raw 32-row tile is 18 KB of consecutive 1 KB DMA chunks (wave w:
  // chunks w, w+NW, ...); lane l of chunk q copies bytes [1024q + 16l, +16) of
  // the tile, i.e. part of row (1024q + 16l) / 576.  The last wave also copies
  // the 32 row scales.
  // lane l of chunk k (k-th chunk of this wave, q = wv + NW*k) copies bytes
  // [1024q + 16l, +16) of the tile, part of row (1024q + 16l) / 576; the row
  // ids are read from LDS up front, then each DMA is one instruction
  constexpr int CPW = (kF8Chunks + NW - 1) / NW;   // chunks per wave
  // (the lane index is made opaque here so that the per-lane offsets are
  // formed at each use rather than hoisted out of the tile loop, where they
  // would hold registers for the whole loop)
  auto raw_ids = [&](int tile, int (&rk)[CPW], int &rid) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
      const int q = wv + NW * k;
      rk[k] = q < kF8Chunks ? row_id(32 * tile + (1024 * q + 16 * ln) / kF8Row) : 0x7fffffff;
    }
    rid = (wv == NW - 1 && ln < 32) ? row_id(32 * tile + ln) : 0x7fffffff;
  };
  auto raw_chunk = [&](int k, int rkk, uint8_t *R) {
    const int q = wv + NW * k;
    if (q < kF8Chunks && rkk != 0x7fffffff) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int o = 1024 * q + 16 * ln, row = o / kF8Row;
      const uint8_t *rp = rkk >= 0 ? wbase + (int64_t)rkk * RB : pbase + (int64_t)(-1 - rkk) * RB;
      __builtin_amdgcn_global_load_lds(rp + (o - row * kF8Row), (lds_void *)(R + 1024 * q), 16, 0, 0);
    }
  };
  auto raw_scale = [&](int rid, float *Sc) {
    if (rid != 0x7fffffff) {
      const float *sp = rid >= 0 ? wsc + rid : psc + (-1 - rid);
      __builtin_amdgcn_global_load_lds(sp, (lds_void *)Sc, 4, 0, 0);
    }
  };
  auto gather_raw = [&](int tile, uint8_t *R, float *Sc) {
    int rk[CPW], rid;
    raw_ids(tile, rk, rid);
#pragma unroll
    for (int k = 0; k < CPW; ++k) raw_chunk(k, rk[k], R);
    raw_scale(rid, Sc);
  };
  // FP8: decode raw tile buf into the fp16 tile T.  Thread t takes row t/8 (of
  // 32) and its 8-channel columns t%8 + 8i: seven of E4M3 codes, one of bf16
  // rope channels, so every LDS address is a per-thread base plus a constant.
  auto convert = [&](const uint8_t *R, const float *sc, uint16_t *T) {
    static_assert(kF8Nope == 56 * 8, "7 E4M3 columns + 1 rope column per thread");
    int t8 = tid;
    asm volatile("" : "+v"(t8));   // formed at each use, not held across the tile loop
    const int j8 = t8 & 7;
#pragma unroll
    for (int row = t8 >> 3; row < 32; row += NT / 8) {
      const uint8_t *rr = R + row * kF8Row + 8 * j8;
      uint16_t *tr = T + row * KP + 8 * j8;
      // s = m 2^e: the conversion applies 2^e exactly (E4M3 values are exact in
      // fp16), one fp16 multiply applies m in [1, 2)
      const float s = sc[row];
      const _Float16 m = (_Float16)__uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
      const h2 mm = h2{m, m};
      u32x2 v[7];
#pragma unroll
      for (int i = 0; i < 7; ++i) v[i] = *reinterpret_cast<const u32x2 *>(rr + 64 * i);
      const u32x4 rv = *reinterpret_cast<const u32x4 *>(R + row * kF8Row + kF8Nope + 16 * j8);
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        const h2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i].x, s, false) * mm;
        const h2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i].x, s, true) * mm;
        const h2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i].y, s, false) * mm;
        const h2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v[i].y, s, true) * mm;
        uint32_t w[4];
        __builtin_memcpy(&w[0], &a0, 4);
        __builtin_memcpy(&w[1], &a1, 4);
        __builtin_memcpy(&w[2], &a2, 4);
        __builtin_memcpy(&w[3], &a3, 4);
        *reinterpret_cast<u32x4 *>(tr + 64 * i) = u32x4{w[0], w[1], w[2], w[3]};
      }
      *reinterpret_cast<u32x4 *>(T + row * KP + kF8Nope + 8 * j8) =
          u32x4{bf16x2_to_f16x2(rv.x), bf16x2_to_f16x2(rv.y), bf16x2_to_f16x2(rv.z), bf16x2_to_f16x2(rv.w)};
    }
  };

  // q~ = RoPE(q) * sm_scale * log2(e) in fp16, B operand: head h0 + 16hb + c,
  // dims 32j + 8g .. +8; the raw loads were issued before the setup work
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int d0 = 32 * j + 8 * g;
      u32x4 raw;
      __builtin_memcpy(&raw, &qb[hb][j], 16);
      float x[8];
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[2 * k] = bf16_to_f32((uint16_t)(wds[k] & 0xFFFF));
        x[2 * k + 1] = bf16_to_f32((uint16_t)(wds[k] >> 16));
      }
      if (d0 >= D - R) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int pi = (d0 + 2 * k - (D - R)) >> 1;
          const float cs = rc[pi], sn = rs[pi];
          const float a = x[2 * k] * cs - x[2 * k + 1] * sn, bb = x[2 * k] * sn + x[2 * k + 1] * cs;
          x[2 * k] = a;
          x[2 * k + 1] = bb;
        }
      }
      const u32x4 o = u32x4{pack_f16x2(x[0] * A.scale_log2, x[1] * A.scale_log2),
                            pack_f16x2(x[2] * A.scale_log2, x[3] * A.scale_log2),
                            pack_f16x2(x[4] * A.scale_log2, x[5] * A.scale_log2),
                            pack_f16x2(x[6] * A.scale_log2, x[7] * A.scale_log2)};
      __builtin_memcpy(&qb[hb][j], &o, 16);
    }
  }

  f32x4 acc_o[AH][DB];
  float m_ref[NHB], m_seen[NHB], l_run[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) { m_ref[hb] = -INFINITY; m_seen[hb] = -INFINITY; }

  // one tile: scores, probabilities against m_ref (raised within the tile when
  // a logit passes it by more than 2^15), PV.
  // Tn/idn: the next tile's buffer and row ids (Tn == nullptr: nothing to
  // gather); its DMAs are spread over the k-steps of S^T so that their issue
  // (the texture path moves 64 B per clock per CU) overlaps the matrix cores
  auto compute = [&](const uint16_t *__restrict__ T, int tile, uint16_t *__restrict__ Tn, uint64_t idn,
                     uint8_t *__restrict__ Rn, float *__restrict__ Sn, int ntile) {
    const int base = 32 * tile;
    // FP8 rows: the next raw tile's gather is issued during this tile's
    // matrix work (its buffer is disjoint from T), one DMA per few k-steps
    int grk[FP8 ? CPW : 1], grid_ = 0x7fffffff;
    if constexpr (FP8) {
      if (Rn) {
        raw_ids(ntile, grk, grid_);
        raw_scale(grid_, Sn);
        // dimension-split path: the whole raw tile at once, so that its
        // latency has the full tile to hide behind
        if constexpr (DSPV) {
#pragma unroll
          for (int k = 0; k < CPW; ++k) raw_chunk(k, grk[k], Rn);
        }
      }
    }
    f32x4 s[NHB][2];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) { s[hb][0] = f32x4{0.f, 0.f, 0.f, 0.f}; s[hb][1] = s[hb][0]; }
    // S^T = K q~^T, software-pipelined QD k-steps deep; the scheduling barriers
    // keep the compiler from hoisting every LDS read at once
    {
      constexpr int QD = DSPV ? 3 : 2;   // k-steps of K prefetch (registers left after the accumulators)
      const uint16_t *k0 = T + c * KP + 8 * g;
      const uint16_t *k1 = k0 + 16 * KP;
      f16x8 r0[QD], r1[QD];
#pragma unroll
      for (int j = 0; j < QD; ++j) {
        r0[j] = *reinterpret_cast<const f16x8 *>(k0 + 32 * j);
        r1[j] = *reinterpret_cast<const f16x8 *>(k1 + 32 * j);
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const f16x8 a0 = r0[j % QD], a1 = r1[j % QD];
        if (j + QD < NJ) {
          r0[j % QD] = *reinterpret_cast<const f16x8 *>(k0 + 32 * (j + QD));
          r1[j % QD] = *reinterpret_cast<const f16x8 *>(k1 + 32 * (j + QD));
        }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          s[hb][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qb[hb][j], s[hb][0], 0, 0, 0);
          s[hb][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qb[hb][j], s[hb][1], 0, 0, 0);
        }
        if (!DSPV && Tn) {
#pragma unroll
          for (int k = (j * RPW) / NJ; k < ((j + 1) * RPW) / NJ; ++k) dma_row(idn, k, Tn);
        }
        if constexpr (FP8 && !DSPV) {
          if (Rn) {
#pragma unroll
            for (int k = (j * CPW) / NJ; k < ((j + 1) * CPW) / NJ; ++k) raw_chunk(k, grk[k], Rn);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // probabilities of head block hb against its reference, packed as the P^T fragment
    auto probs = [&](int hb, f16x8 &pf) -> float {
      float p[8], psum = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[4 * mb + i] = __builtin_amdgcn_exp2f(s[hb][mb][i] - m_ref[hb]);
          psum += p[4 * mb + i];
        }
      const u32x4 pw = u32x4{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3]), pack_f16x2(p[4], p[5]),
                             pack_f16x2(p[6], p[7])};
      __builtin_memcpy(&pf, &pw, 16);
      return psum;
    };
    uint32_t raised = 0;
    f16x8 pb[NHB];
    float ps[NHB];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      if (base + 32 > nrows) {   // only the last tile holds positions past the list
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (base + 16 * mb + 4 * g + i >= nrows) s[hb][mb][i] = -INFINITY;
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mloc = fmaxf(mloc, s[hb][mb][i]);
      mloc = rows_max(mloc);
      m_seen[hb] = fmaxf(m_seen[hb], mloc);
      if (m_ref[hb] == -INFINITY) m_ref[hb] = mloc;   // first tile
      // the wave owns its heads' whole tile: a logit more than 2^15 above the
      // reference raises the reference to the largest logit seen, and the
      // running sum and the accumulators follow by 2^(old - new) (DSPV: the
      // accumulators of these heads are spread over every wave, so the factor
      // goes to the others through LDS with the P^T fragment)
      if (__ballot(mloc > m_ref[hb] + kRefSlack)) {
        const float f = __builtin_amdgcn_exp2f(m_ref[hb] - m_seen[hb]);
        m_ref[hb] = m_seen[hb];
        l_run[hb] *= f;
        if constexpr (!DSPV) {
#pragma unroll
          for (int db = 0; db < DB; ++db) acc_o[hb][db] = acc_o[hb][db] * f;
        } else {
          if (g == 0) fsh[16 * wv + c] = f;
          raised = 1;
        }
        if (A.diag && lane == 0) atomicAdd(&g_diag[DSV4_DIAG_REF_RAISES], 1ull);
      }
      ps[hb] = probs(hb, pb[hb]);
      l_run[hb] += ps[hb];
    }
    if constexpr (DSPV) {
      // every wave's P^T fragment to LDS (PB was last read before the previous
      // tile's closing barrier), then O^T[this wave's channels, all heads]
      *reinterpret_cast<f16x8 *>(PB + (wv * 64 + lane) * 8) = pb[0];
      if (lane == 0) reinterpret_cast<uint8_t *>(&rfl)[wv] = (uint8_t)raised;   // read after the barrier
      // the next tile's gather: issued where the wave would wait for the others'
      // scores anyway (its buffer was released by the previous tile's closing barrier)
      if (!FP8 && Tn) {
#pragma unroll
        for (int k = 0; k < RPW; ++k) dma_row(idn, k, Tn);
      }
      lds_barrier();   // P^T of every wave visible; the next tile's DMAs stay in flight
      // the accumulators of heads whose reference rose in this tile follow it
      // (the flags and P^T are rewritten only after the tile's closing barrier)
      if (const uint32_t fl = rfl) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          if ((fl >> (8 * w)) & 0xffu) {
            const float fw = fsh[16 * w + c];
#pragma unroll
            for (int db = 0; db < DB; ++db) acc_o[w][db] = acc_o[w][db] * fw;
          }
        }
      }
      // the running sum and maximum settled here, so no probability stays live across PV
      asm volatile("" : "+v"(l_run[0]), "+v"(m_seen[0]));
      // head blocks in groups of HG (P^T fragments live: HG; V^T read NW/HG times)
      constexpr int HG = NW;
      const uint16_t *v0p = T + (4 * g + (c >> 2)) * KP + 4 * (c & 3) + 16 * wv;
      const uint16_t *v1p = v0p + 16 * KP;
#pragma unroll
      for (int w0 = 0; w0 < NW; w0 += HG) {
        f16x8 pw[HG];
#pragma unroll
        for (int w = 0; w < HG; ++w) pw[w] = *reinterpret_cast<const f16x8 *>(PB + ((w0 + w) * 64 + lane) * 8);
        constexpr int VD = 4;
        v4i16 vlo[VD], vhi[VD];
#pragma unroll
        for (int db = 0; db < VD; ++db) {
          vlo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v0p + 16 * CS * db));
          vhi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v1p + 16 * CS * db));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          f16x8 a;
          __builtin_memcpy(&a, &vlo[db % VD], 8);
          __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &vhi[db % VD], 8);
          if (db + VD < DB) {
            vlo[db % VD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v0p + 16 * CS * (db + VD)));
            vhi[db % VD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v1p + 16 * CS * (db + VD)));
          }
#pragma unroll
          for (int w = 0; w < HG; ++w)
            acc_o[w0 + w][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pw[w], acc_o[w0 + w][db], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      return;
    }
    // O^T += V^T P^T; V^T fragments by transposing reads of the row-major tile,
    // pipelined VD 16-dim blocks deep
    constexpr int VD = 3;
    const uint16_t *v0p = T + (4 * g + (c >> 2)) * KP + 4 * (c & 3);
    const uint16_t *v1p = v0p + 16 * KP;
    v4i16 vlo[VD], vhi[VD];
#pragma unroll
    for (int db = 0; db < VD; ++db) {
      vlo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v0p + 16 * db));
      vhi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v1p + 16 * db));
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      f16x8 a;
      __builtin_memcpy(&a, &vlo[db % VD], 8);
      __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &vhi[db % VD], 8);
      if (db + VD < NDB) {
        vlo[db % VD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v0p + 16 * (db + VD)));
        vhi[db % VD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v1p + 16 * (db + VD)));
      }
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb)
        if constexpr (!DSPV) acc_o[hb][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb[hb], acc_o[hb][db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  {
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) l_run[hb] = 0.f;
#pragma unroll
    for (int ah = 0; ah < AH; ++ah)
#pragma unroll
      for (int db = 0; db < DB; ++db) acc_o[ah][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    int it = 0;
    if constexpr (!FP8) {
      if (tile_lo < tile_hi && !early) gather(tile_lo, T0);
      vm_wait_all();     // this wave's rows of the first tile landed ...
      __syncthreads();   // ... and every wave's
      for (int tile = tile_lo; tile < tile_hi; ++tile, ++it) {
        const bool odd = it & 1;
        const bool more = tile + 1 < tile_hi;
        compute(odd ? T1 : T0, tile, more ? (odd ? T0 : T1) : nullptr, more ? tile_addr(tile + 1) : 0, nullptr,
                nullptr, 0);
        vm_wait_all();     // this wave's rows of the next tile landed ...
        __syncthreads();   // ... and every wave's; this one fully read
      }
    } else {
      // one raw buffer and one fp16 tile (two workgroups share a CU, so one's
      // waits overlap the other's matrix work): raw tile i+1 is gathered
      // during compute(i), then decoded into the tile compute(i) just read
      if (tile_lo < tile_hi) gather_raw(tile_lo, RW, RSC);
      vm_wait_all();     // this wave's part of the raw tile landed ...
      __syncthreads();   // ... and every wave's
      if (tile_lo < tile_hi) convert(RW, RSC, T0);
      lds_barrier();
      for (int tile = tile_lo; tile < tile_hi; ++tile, ++it) {
        const bool more = tile + 1 < tile_hi;
        compute(T0, tile, nullptr, 0, more ? RW : nullptr, RSC, tile + 1);
        vm_wait_all();     // this wave's part of raw tile+1 landed ...
        __syncthreads();   // ... and every wave's; the tile fully read
        if (more) convert(RW, RSC, T0);
        lds_barrier();
      }
    }
  }

  // DSPV: the head-owning waves' (reference, sum) pairs through LDS
  float *shml = reinterpret_cast<float *>(PB);
  if constexpr (DSPV) {
    const float lr = rows_sum(l_run[0]);
    if (g == 0) {
      shml[2 * (16 * wv + c)] = m_ref[0];
      shml[2 * (16 * wv + c) + 1] = lr;
    }
    __syncthreads();
  }
  // bf16 outputs of the dimension-split path are staged in the (now idle) tile
  // buffers, heads as rows, so that every global store writes one whole 1 KB row.
  // The output form is chosen once (MD: 0 split partials, 1 staged bf16, 2 fp32,
  // 3 bf16), not per channel block.
  auto finish = [&](auto MDc) {
    constexpr int MD = decltype(MDc)::value;
#pragma unroll
    for (int hb = 0; hb < AH; ++hb) {
      const int h = DSPV ? 16 * hb + c : h0 + 16 * hb + c;
      float lr, mr;
      if constexpr (DSPV) {
        mr = shml[2 * h];
        lr = shml[2 * h + 1];
      } else {
        lr = l_run[hb];
        lr += __shfl_xor(lr, 16, 64);
        lr += __shfl_xor(lr, 32, 64);
        mr = m_ref[hb];
      }
      const int dlo = DSPV ? 16 * wv : 0;   // this wave's first output channel
      if constexpr (MD == 0) {
        const int64_t pr = ((int64_t)r * e_ns + split) * e_H + h;
        uint16_t *po = e_po + pr * D;
        const float inv = lr > 0.f ? 1.f / lr : 0.f;   // normalised: within the rows' range, fp16-safe
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 a = acc_o[hb][db];
          *reinterpret_cast<u32x2 *>(po + dlo + 16 * CS * db + 4 * g) =
              u32x2{pack_f16x2(a[0] * inv, a[1] * inv), pack_f16x2(a[2] * inv, a[3] * inv)};
        }
        if (g == 0 && (!DSPV || hb == wv)) {
          e_pml[2 * pr] = mr;
          e_pml[2 * pr + 1] = lr;
        }
      } else {
        // the sink joins the denominator; both exponents are <= 0 (hardware exp2,
        // reciprocal within an ulp: far below the output's bf16 rounding)
        float f = 1.f, den = lr;
        if (e_sk) {
          const float sg = sk[h];
          const float M = fmaxf(mr, sg);
          f = __builtin_amdgcn_exp2f(mr - M);
          den = lr * f + __builtin_amdgcn_exp2f(sg - M);
        }
        const float inv = den > 0.f ? f * __builtin_amdgcn_rcpf(den) : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          float o[4];
          const int d0 = dlo + 16 * CS * db + 4 * g;
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = acc_o[hb][db][i] * inv;
          if (d0 >= D - R) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const int pi = (d0 + 2 * k - (D - R)) >> 1;
              const float cs = rc[pi], sn = rs[pi];
              const float a = o[2 * k] * cs + o[2 * k + 1] * sn, bb = -o[2 * k] * sn + o[2 * k + 1] * cs;
              o[2 * k] = a;
              o[2 * k + 1] = bb;
            }
          }
          const int64_t oe = ((int64_t)r * e_H + h) * D + d0;
          if constexpr (MD == 1) {
            *reinterpret_cast<u32x2 *>((h < 32 ? T0 : T1) + (h & 31) * KP + d0) =
                u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          } else if constexpr (MD == 2) {
            *reinterpret_cast<f32x4 *>((float *)A.out + oe) = f32x4{o[0], o[1], o[2], o[3]};
          } else {
            *reinterpret_cast<u32x2 *>((uint16_t *)A.out + oe) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          }
        }
      }
    }
  };
  if (e_ns > 1) finish(std::integral_constant<int, 0>{});
  else if (stage) finish(std::integral_constant<int, 1>{});
  else if (e_odt == DSV4_F32) finish(std::integral_constant<int, 2>{});
  else finish(std::integral_constant<int, 3>{});
  if (stage) {
    __syncthreads();
    // wave w writes the rows of heads 16w .. 16w+15: lane l carries channels 8l .. 8l+7
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      const int h = 16 * wv + k;
      const u32x4 v = *reinterpret_cast<const u32x4 *>((h < 32 ? T0 : T1) + (h & 31) * KP + 8 * lane);
      *reinterpret_cast<u32x4 *>(orow + h * D + 8 * lane) = v;
    }
  }
}

// ---------------------------------------------------------------- FP8 rows, decode
// k_attn_dec<NHB, R64>: the decode form of the FP8-row path (one query row per
// sequence, its row list split over several workgroups), for H = 16 NHB heads.
// Two waves per SIMD: 2 NHB waves, wave w = (head block w % NHB, row half
// w / NHB).  Per 32-row tile:
//   * S^T = K q~^T: each wave scores its 16 rows against its 16 heads (the K
//     fragments it reads from LDS are half a tile, so the tile's LDS reads are
//     spread over twice the waves);
//   * the fixed-reference softmax: both row halves of a head share one
//     reference, taken from the first tile with a valid row through one LDS
//     exchange (and raised inside a tile, with the partial sums and the
//     accumulators rescaled, when a logit passes it by more than 2^15); each
//     wave publishes its 16-row half of the head block's P^T fragment;
//   * O^T = V^T P^T with the channels split over all waves (wave w owns the
//     16-channel blocks w, w + 2 NHB, ...), every P^T fragment read by every
//     wave, so each V^T fragment read from LDS feeds NHB products.
// Around it, a pipeline made for short row lists that live in HBM:
//   * the query's picks, sinks and rope frequencies are loaded first and the
//     query row after them, so the gathers wait for the picks only; the query
//     row is converted to q~ once per workgroup (each thread 1/NT of it) and
//     handed to the waves through LDS, overlapping the first gathers;
//   * no index compaction: a split keeps the picks of its own tiles, and a
//     pick that is -1 or past the pool count is a masked row (its tile row is
//     written as zeros, its probability is zero);
//   * gathers into registers, two tiles ahead: sixteen threads per row, each
//     loading 28 bytes of E4M3 codes, 8 bytes of bf16 rope channels and the
//     row scale, then decoding them into one of two fp16 tiles itself, so the
//     raw rows never pass through LDS and no wave waits on another's loads; a
//     gather past the split's last tile reads a row that exists, so every step
//     issues the same loads and the compiler's waits stay exact;
//   * two barriers per tile: P^T published, and the next fp16 tile written;
//   * the splits of one query sit on one XCD (workgroups are dealt to the
//     eight XCDs in turn), so its query row and picks come into one L2;
//   * split partials (fp16, normalised by the split's own sum) and bf16
//     outputs are staged in LDS, heads as rows, so each store writes a whole
//     1 KB head row.
// Decoding E4M3 with scale s = m 2^e: the conversion applies 2^e exactly
// (E4M3 values are exact in fp16), one fp16 multiply applies m in [1, 2).
template <int NHB>
struct DecRaw {
  static constexpr int NT = 128 * NHB;
  static constexpr int RPT = 512 / NT;   // tile rows a thread gathers (16 threads per row)
  u32x4 a[RPT];                          // E4M3 bytes [28p, 28p + 16) of the row
  u32x2 b[RPT];                          // [28p + 16, 28p + 24)
  uint32_t c[RPT];                       // [28p + 24, 28p + 28)
  u32x2 rp[RPT];                         // rope bytes [448 + 8p, +8): four bf16 channels
  float s[RPT];
  uint32_t ok;                           // bit q: row q of this thread is valid
};

// read in place of absent sinks (never written; the value read is not used),
// global memory like the sinks so that the read is a global load
__device__ float kNoSinks[64];

// an unaligned global load of a T (the addresses here are 4-byte aligned)
template <class T>
__device__ __forceinline__ T ldg_u(const uint8_t *p) {
  T v;
  __builtin_memcpy(&v, p, sizeof(T));
  return v;
}

// bits 0, 16, 32, 48 of a wave ballot (lane 16k stands for row k of 4) as 4 bits
__device__ __forceinline__ uint32_t row_bits4(uint64_t b) {
  return (uint32_t)(b & 1u) | (uint32_t)((b >> 15) & 2u) | (uint32_t)((b >> 30) & 4u) | (uint32_t)((b >> 45) & 8u);
}

template <int NHB, bool R64>
__global__ __launch_bounds__(128 * NHB, 1) void k_attn_dec(AttnArgs A) {
  constexpr int D = 512, KP = D + 16, NJ = D / 32, NDB = D / 16;
  constexpr int NWV = 2 * NHB, NT = 64 * NWV;   // waves, threads
  constexpr int RB = kF8Row;
  constexpr int DBW = NDB / NWV;                // 16-channel blocks per wave in PV
  constexpr int RPT = DecRaw<NHB>::RPT;
  constexpr int RSTEP = NT / 16;                // between a thread's rows
  constexpr int TH = 32 * KP;                   // halfs per fp16 tile
  constexpr int QP = D + 8;                     // staged q~ row pitch (halfs)
  constexpr int SROW = 1040;                    // staged output row pitch (bytes)
  static_assert(NHB == 1 || NHB == 2 || NHB == 4, "16, 32 or 64 heads");
  static_assert(RPT * RSTEP == 32, "a gather covers the tile");
  static_assert(2 * TH * 2 >= 16 * NHB * SROW && 2 * TH >= 16 * NHB * QP, "staging fits in the tile buffers");
  __shared__ __attribute__((aligned(16))) uint16_t TT[2 * TH];   // two fp16 tiles
  __shared__ uint32_t vmk[4][NWV];   // valid rows of tile t, slot t % 4: one field per wave
  __shared__ int ids[kMaxSel];       // this split's picks
  __shared__ float rc[32], rs[32];
  __shared__ float sk[64];
  __shared__ float xm[2][64];        // per row half: a head's tile maximum, then its sum
  __shared__ float fsh[64];          // per-head factors of a reference raise
  __shared__ int rflag[3];
  __shared__ __attribute__((aligned(16))) uint16_t PB[NHB * 64 * 8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int hb = wv % NHB, rh = wv / NHB;   // this wave's head block and row half
  int L = (int)blockIdx.x;
  if ((gridDim.x & 7u) == 0) L = (int)((blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3));
  const int r = (A.T - 1) - L / A.nsplit;
  const int split = L % A.nsplit;

  // the picks (clamped reads, so the count of loads is fixed), the sinks and
  // the rope frequencies first; the query row after them
  constexpr int IPT = (kMaxSel + NT - 1) / NT;
  int ipre[IPT];
  if (A.csa && A.topk > 0) {
    const int32_t *ix = A.idx + (int64_t)r * A.topk;
#pragma unroll
    for (int k = 0; k < IPT; ++k) ipre[k] = ix[min(tid + NT * k, A.topk - 1)];
  }
  const float sink = (A.sinks ? A.sinks : kNoSinks)[min(tid, A.H - 1)];   // one unconditional load
  const double ifq = A.inv_freq[tid & 31];
  // the query row in 8-channel chunks: thread t holds plain chunks t + NT i
  // (i < 7, numbered over the 56 non-rope chunks of each head) and the rope
  // chunk t (head t / 8, channels 448 + 8 (t % 8)), so that every wave does
  // the same work for every chunk it converts
  static_assert(16 * NHB * (D / 8) == 8 * NT, "eight chunks per thread");
  f16x8 qb[8];
  {
    const uint16_t *qr = (const uint16_t *)A.q + (int64_t)r * A.H * D;
#pragma unroll
    for (int i = 0; i < 7; ++i) {
      const int k = tid + NT * i;
      qb[i] = *reinterpret_cast<const f16x8 *>(qr + (k / 56) * D + 8 * (k % 56));
    }
    qb[7] = *reinterpret_cast<const f16x8 *>(qr + (tid >> 3) * D + (D - 64) + 8 * (tid & 7));
  }
  RowPlan P = row_plan(A, r);
  const int R = R64 ? 64 : A.rope_dim;
  const int nwin = P.nwin, csa = A.csa;
  const int pcount = P.pcount;
  // nominal row list: window rows, then every pick slot (CSA) or the visible entries (HCA)
  const int nrows = nwin + (csa ? A.topk : P.nsel);
  const int ntiles = (nrows + 31) / 32;
  const int tps = (ntiles + A.nsplit - 1) / A.nsplit;
  const int tile_lo = split * tps;
  int tile_hi = min(ntiles, tile_lo + tps);
  const int e_lo = max(0, 32 * tile_lo - nwin), e_hi = csa ? min(A.topk, 32 * tile_hi - nwin) : 0;
  if (csa && A.topk > 0) {
    unsigned long long nb = 0;
#pragma unroll
    for (int k = 0; k < IPT; ++k) {
      const int e = tid + NT * k;
      if (e >= e_lo && e < e_hi) {
        ids[e - e_lo] = ipre[k];
        nb += (ipre[k] != -1 && !(ipre[k] >= 0 && ipre[k] < pcount)) ? 1ull : 0ull;
      }
    }
    if (A.diag && nb) atomicAdd(&g_diag[DSV4_DIAG_BAD_PICKS], nb);
  }
  const uint8_t *pbase = A.pool.data ? A.pool.data + (int64_t)P.b * A.pool.stride * RB : nullptr;
  const uint8_t *wbase = A.win.data ? A.win.data + (int64_t)P.b * A.win.stride * RB : nullptr;
  const float *psc = A.pool.data ? A.pool.rscale + (int64_t)P.b * A.pool.stride : nullptr;
  const float *wsc = A.win.data ? A.win.rscale + (int64_t)P.b * A.win.stride : nullptr;
  // every invalid position reads a row that exists (its values are replaced by
  // zeros): the first window row, else pool entry 0; with neither there is no row
  if (!(nwin > 0 || pcount > 0)) tile_hi = tile_lo;
  if (tid < R / 2) rope_cs_f((double)P.p, ifq, 1.f, &rc[tid], &rs[tid]);
  if (tid < A.H) sk[tid] = A.sinks ? sink * kLog2e : -INFINITY;
  if (tid < 3) rflag[tid] = 0;
  lds_barrier();   // picks, angles and sinks visible; the query row may still be in flight

  // row i of the list: its address and scale address, and whether it is valid
  auto row_src = [&](int i, const uint8_t **rp, const float **sp) -> bool {
    bool ok = i >= 0 && i < nrows;
    int wrow = -1, pent = -1;
    if (ok && i < nwin) wrow = win_slot(A, P, i);
    else if (ok) {
      pent = csa ? ids[i - nwin - e_lo] : i - nwin;
      ok = pent >= 0 && pent < pcount;
    }
    if (!ok) {   // the row every invalid position reads
      wrow = nwin > 0 ? win_slot(A, P, 0) : -1;
      pent = nwin > 0 ? -1 : 0;
    }
    *rp = wrow >= 0 ? wbase + (int64_t)wrow * RB : pbase + (int64_t)pent * RB;
    *sp = wrow >= 0 ? wsc + wrow : psc + pent;
    return ok;
  };
  // gather tile t (t < 0: no tile, every row reads the stand-in row) into
  // registers; the rows' validity goes to this wave's field of vmk
  const int p16 = tid & 15;
  auto gather = [&](int t, DecRaw<NHB> &Rw) {
    uint32_t wm = 0;
    Rw.ok = 0;
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int row = (tid >> 4) + q * RSTEP;
      const uint8_t *rp = nullptr;
      const float *sp = nullptr;
      const bool ok = row_src(t >= 0 ? 32 * t + row : -1, &rp, &sp);
      Rw.ok |= (uint32_t)ok << q;
      const uint8_t *p8 = rp + 28 * p16;
      Rw.a[q] = ldg_u<u32x4>(p8);
      Rw.b[q] = ldg_u<u32x2>(p8 + 16);
      Rw.c[q] = ldg_u<uint32_t>(p8 + 24);
      Rw.rp[q] = ldg_u<u32x2>(rp + kF8Nope + 8 * p16);
      Rw.s[q] = *sp;
      wm |= row_bits4(__ballot(ok)) << (4 * wv + q * RSTEP);
    }
    if (t >= 0 && lane == 0) vmk[t & 3][wv] = wm;
  };
  auto tile_mask = [&](int t) {
    uint32_t m = 0;
#pragma unroll
    for (int w = 0; w < NWV; ++w) m |= vmk[t & 3][w];
    return m;
  };
  // gathered registers -> fp16 tile Tb (invalid rows become zeros)
  auto convert = [&](const DecRaw<NHB> &Rw, uint16_t *Tb) {
#pragma unroll
    for (int q = 0; q < RPT; ++q) {
      const int row = (tid >> 4) + q * RSTEP;
      uint16_t *tr = Tb + row * KP + 28 * p16;
      uint16_t *tq = Tb + row * KP + kF8Nope + 4 * p16;
      // the row's loads have landed on every path through the branch below,
      // so the compiler's waits stay exact (one tile of gathers in flight)
      asm volatile("" ::"v"(Rw.a[q]), "v"(Rw.b[q]), "v"(Rw.c[q]), "v"(Rw.rp[q]), "v"(Rw.s[q]));
      if (!((Rw.ok >> q) & 1u)) {
#pragma unroll
        for (int i = 0; i < 7; ++i) *reinterpret_cast<u32x2 *>(tr + 4 * i) = u32x2{0u, 0u};
        *reinterpret_cast<u32x2 *>(tq) = u32x2{0u, 0u};
        continue;
      }
      const float s = Rw.s[q];
      const _Float16 m = (_Float16)__uint_as_float((__float_as_uint(s) & 0x007FFFFFu) | 0x3F800000u);
      const h2 mm = h2{m, m};
      const uint32_t wd[7] = {Rw.a[q].x, Rw.a[q].y, Rw.a[q].z, Rw.a[q].w, Rw.b[q].x, Rw.b[q].y, Rw.c[q]};
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        const h2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd[i], s, false) * mm;
        const h2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wd[i], s, true) * mm;
        uint32_t w0, w1;
        __builtin_memcpy(&w0, &lo, 4);
        __builtin_memcpy(&w1, &hi, 4);
        *reinterpret_cast<u32x2 *>(tr + 4 * i) = u32x2{w0, w1};
      }
      *reinterpret_cast<u32x2 *>(tq) = u32x2{bf16x2_to_f16x2(Rw.rp[q].x), bf16x2_to_f16x2(Rw.rp[q].y)};
    }
  };

  DecRaw<NHB> R0, R1;
  f32x4 acc_o[NHB][DBW];
  float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
  auto clear_acc = [&]() {
#pragma unroll
    for (int h = 0; h < NHB; ++h)
#pragma unroll
      for (int db = 0; db < DBW; ++db) acc_o[h][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  // everything up to the epilogue sits in one branch, so that the compiler's
  // load waits see a single path: the q~ conversion waits for the query row
  // only, with the first two gathers still in flight behind it
  if (tile_lo < tile_hi) {
  gather(tile_lo, R0);
  gather(tile_lo + 1 < tile_hi ? tile_lo + 1 : -1, R1);
  // q~ = RoPE(q) * sm_scale * log2(e) in fp16, staged in the tile buffers as
  // head rows; then each wave takes its B operand (head 16 hb + c, dims 32j + 8g .. +8)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int k = tid + NT * i;
    const int h = i < 7 ? k / 56 : tid >> 3, d0 = i < 7 ? 8 * (k % 56) : (D - 64) + 8 * (tid & 7);
    u32x4 raw;
    __builtin_memcpy(&raw, &qb[i], 16);
    float x[8];
    const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16_to_f32((uint16_t)(wds[k] & 0xFFFF));
      x[2 * k + 1] = bf16_to_f32((uint16_t)(wds[k] >> 16));
    }
    if (i == 7 && d0 >= D - R) {   // the rope chunk (R <= 64)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int pi = (d0 + 2 * k - (D - R)) >> 1;
        const float cs = rc[pi], sn = rs[pi];
        const float a = x[2 * k] * cs - x[2 * k + 1] * sn, bb = x[2 * k] * sn + x[2 * k + 1] * cs;
        x[2 * k] = a;
        x[2 * k + 1] = bb;
      }
    }
    *reinterpret_cast<u32x4 *>(TT + h * QP + d0) =
        u32x4{pack_f16x2(x[0] * A.scale_log2, x[1] * A.scale_log2), pack_f16x2(x[2] * A.scale_log2, x[3] * A.scale_log2),
              pack_f16x2(x[4] * A.scale_log2, x[5] * A.scale_log2), pack_f16x2(x[6] * A.scale_log2, x[7] * A.scale_log2)};
  }
  lds_barrier();
  f16x8 qf[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) qf[j] = *reinterpret_cast<const f16x8 *>(TT + (16 * hb + c) * QP + 32 * j + 8 * g);
  lds_barrier();   // every wave holds its q~ fragments: the tile buffers are free
  clear_acc();

  bool ref_set = false;   // the reference of this pass is taken (uniform over the workgroup)
  // one tile on the matrix cores (fp16 tile Tb).  A logit far above the
  // reference sets rflag[fl].
  auto compute = [&](const uint16_t *Tb, int tile, int fl) {
    const uint32_t mask = tile_mask(tile);
    f32x4 s0 = f32x4{0.f, 0.f, 0.f, 0.f}, s1 = s0;   // even and odd k-steps: two MFMA chains
    {
      constexpr int QD = 4;
      const uint16_t *k0 = Tb + (16 * rh + c) * KP + 8 * g;
      f16x8 r0[QD];
#pragma unroll
      for (int j = 0; j < QD; ++j) r0[j] = *reinterpret_cast<const f16x8 *>(k0 + 32 * j);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const f16x8 a0 = r0[j % QD];
        if (j + QD < NJ) r0[j % QD] = *reinterpret_cast<const f16x8 *>(k0 + 32 * (j + QD));
        if (j & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf[j], s1, 0, 0, 0);
        else s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf[j], s0, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float sv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = s0[i] + s1[i];
    if (mask != 0xFFFFFFFFu) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (!((mask >> (16 * rh + 4 * g + i)) & 1u)) sv[i] = -INFINITY;
    }
    float mloc = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mloc = rows_max(mloc);
    m_seen = fmaxf(m_seen, mloc);
    if (!ref_set && mask != 0u) {   // the first tile with a valid row: both halves' maximum
      if (g == 0) xm[rh][16 * hb + c] = mloc;
      lds_barrier();
      m_ref = fmaxf(mloc, xm[1 - rh][16 * hb + c]);
      ref_set = true;
    }
    const bool over = mloc > m_ref + kRefSlack;
    // this wave's 16-row half of the head block's P^T fragment, against the reference
    auto probs = [&]() -> float {
      float p[4], psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[i] - m_ref);
        psum += p[i];
      }
      *reinterpret_cast<u32x2 *>(PB + (hb * 64 + lane) * 8 + 4 * rh) = u32x2{pack_f16x2(p[0], p[1]), pack_f16x2(p[2], p[3])};
      return psum;
    };
    float psum = probs();
    if (__ballot(over) && lane == 0) rflag[fl] = 1;
    lds_barrier();   // P^T of every wave visible
    if (rflag[fl]) {
      // a logit more than 2^15 above its head's reference: every head's
      // reference rises to its largest logit seen so far (both row halves),
      // this tile's P^T is taken again, and the running sums and every wave's
      // accumulators (all heads) scale by 2^(old - new); nothing of this tile
      // has been summed yet
      if (g == 0) xm[rh][16 * hb + c] = m_seen;
      lds_barrier();
      const float mn = fmaxf(m_seen, xm[1 - rh][16 * hb + c]);
      const float f = __builtin_amdgcn_exp2f(m_ref - mn);
      m_ref = mn;
      l_run *= f;
      if (g == 0 && rh == 0) fsh[16 * hb + c] = f;
      psum = probs();
      if (A.diag && tid == 0) atomicAdd(&g_diag[DSV4_DIAG_REF_RAISES], (unsigned long long)NHB);   // every head block rose
      lds_barrier();   // the factors and the new P^T visible
#pragma unroll
      for (int h = 0; h < NHB; ++h) {
        const float fh = fsh[16 * h + c];
#pragma unroll
        for (int db = 0; db < DBW; ++db) acc_o[h][db] = acc_o[h][db] * fh;
      }
    }
    l_run += psum;
    asm volatile("" : "+v"(l_run), "+v"(m_seen));
    const uint16_t *v0p = Tb + (4 * g + (c >> 2)) * KP + 4 * (c & 3) + 16 * wv;
    const uint16_t *v1p = v0p + 16 * KP;
    f16x8 pf[NHB];
#pragma unroll
    for (int h = 0; h < NHB; ++h) pf[h] = *reinterpret_cast<const f16x8 *>(PB + (h * 64 + lane) * 8);
    constexpr int VD = DBW < 4 ? DBW : 4;
    v4i16 vlo[VD], vhi[VD];
#pragma unroll
    for (int db = 0; db < VD; ++db) {
      vlo[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v0p + 16 * NWV * db));
      vhi[db] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v1p + 16 * NWV * db));
    }
#pragma unroll
    for (int db = 0; db < DBW; ++db) {
      f16x8 a;
      __builtin_memcpy(&a, &vlo[db % VD], 8);
      __builtin_memcpy(reinterpret_cast<char *>(&a) + 8, &vhi[db % VD], 8);
      if (db + VD < DBW) {
        vlo[db % VD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v0p + 16 * NWV * (db + VD)));
        vhi[db % VD] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(lds_u16 *)(v1p + 16 * NWV * (db + VD)));
      }
#pragma unroll
      for (int h = 0; h < NHB; ++h) acc_o[h][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pf[h], acc_o[h][db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // tile `tile` (in fp16 tile B, its raw registers free) on the matrix cores
  // while the gather of tile+2 is in flight, then tile+1 decoded into the other
  // fp16 tile.  The gather and the decode run past the last tile too (the
  // stand-in rows decode to zeros; only the matrix work is skipped): with no
  // branch around a load or its use, the compiler's waits for the gathers stay
  // one step deep.
  auto step = [&](auto Bc, int tile, int it) {
    constexpr int B = decltype(Bc)::value;
    DecRaw<NHB> &Rc = B ? R1 : R0;
    DecRaw<NHB> &Rn = B ? R0 : R1;
    gather(tile + 2 < tile_hi ? tile + 2 : -1, Rc);
    if (tile < tile_hi) compute(TT + B * TH, tile, it % 3);
    if (tid == 0) rflag[(it + 1) % 3] = 0;   // last read after the P barrier of tile it-2
    convert(Rn, TT + (1 - B) * TH);
    lds_barrier();   // next fp16 tile written, this one and P^T free
  };
  // the split's tiles, the first two gathers issued.  Tiles go in pairs (an
  // odd count ends with a step that only gathers and decodes), so the loop
  // has one exit point and every path back to its head has passed both
  // steps' waits.
  convert(R0, TT);
  lds_barrier();
  for (int tile = tile_lo, it = 0;; tile += 2, it += 2) {
    step(std::integral_constant<int, 0>{}, tile, it);
    step(std::integral_constant<int, 1>{}, tile + 1, it + 1);
    if (tile + 2 >= tile_hi) break;
  }
  } else {
    clear_acc();
  }

  // every head's (reference, sum over both row halves) through LDS
  {
    const float lr = rows_sum(l_run);
    if (g == 0) xm[rh][16 * hb + c] = lr;
    lds_barrier();
  }
  float *shm = reinterpret_cast<float *>(PB);
  if (rh == 0 && g == 0) {
    shm[2 * (16 * hb + c)] = m_ref;
    shm[2 * (16 * hb + c) + 1] = xm[0][16 * hb + c] + xm[1][16 * hb + c];
  }
  lds_barrier();
  // MODE 0: split partial (fp16, staged), 1: fp32 output (direct), 2: bf16 output (staged)
  auto finish = [&](auto Mc) {
    constexpr int MODE = decltype(Mc)::value;
    const int ns = A.nsplit;
#pragma unroll
    for (int hh = 0; hh < NHB; ++hh) {
      const int h = 16 * hh + c;
      const float mr = shm[2 * h], lr = shm[2 * h + 1];
      float f = 1.f, den = lr;
      if (MODE != 0 && A.sinks) {   // the sink joins the denominator (exponents <= 0)
        const float sg = sk[h];
        const float M = lr > 0.f ? fmaxf(mr, sg) : sg;
        f = lr > 0.f ? __builtin_amdgcn_exp2f(mr - M) : 0.f;
        den = lr * f + __builtin_amdgcn_exp2f(sg - M);
      }
      // split partials: normalised by the split's own sum, so fp16 holds them
      const float inv = den > 0.f ? f * __builtin_amdgcn_rcpf(den) : 0.f;
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        float o[4];
        const int cb = wv + NWV * db, d0 = 16 * cb + 4 * g;
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = acc_o[hh][db][i] * inv;
        if (MODE != 0 && 16 * cb >= D - R) {   // the output's rope slice turns back by -p
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int pi = (d0 + 2 * k - (D - R)) >> 1;
            const float cs = rc[pi], sn = rs[pi];
            const float a = o[2 * k] * cs + o[2 * k + 1] * sn, bb = -o[2 * k] * sn + o[2 * k + 1] * cs;
            o[2 * k] = a;
            o[2 * k + 1] = bb;
          }
        }
        if (MODE == 1) {
          const int64_t oe = ((int64_t)r * A.H + h) * D + d0;
          *reinterpret_cast<f32x4 *>((float *)A.out + oe) = f32x4{o[0], o[1], o[2], o[3]};
        } else {
          const u32x2 v = MODE == 0 ? u32x2{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3])}
                                    : u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          *reinterpret_cast<u32x2 *>(reinterpret_cast<uint8_t *>(TT) + h * SROW + 2 * d0) = v;
        }
      }
      if (MODE == 0 && g == 0 && hh == hb && rh == 0) {
        const int64_t pr = ((int64_t)r * ns + split) * A.H + h;
        A.part_ml[2 * pr] = lr > 0.f ? mr : -INFINITY;
        A.part_ml[2 * pr + 1] = lr;
      }
    }
    if (MODE != 1) {
      lds_barrier();
      // wave w writes the head rows w, w + NWV, ...: lane l carries channels 8l .. 8l+7
      uint16_t *orow = MODE == 0 ? A.part_o + (((int64_t)r * ns + split) * A.H) * D
                                 : (uint16_t *)A.out + (int64_t)r * A.H * D;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int h = wv + NWV * k;
        *reinterpret_cast<u32x4 *>(orow + (int64_t)h * D + 8 * lane) =
            *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint8_t *>(TT) + h * SROW + 16 * lane);
      }
    }
  };
  if (A.nsplit > 1) finish(std::integral_constant<int, 0>{});
  else if (A.out_dtype == DSV4_F32) finish(std::integral_constant<int, 1>{});
  else finish(std::integral_constant<int, 2>{});
}

// Merge split partials: grid (T * H), block D/2 threads (one channel pair each).
// Every load that does not depend on another (the channel pair of every split,
// the splits' (max, sum)) is issued first, so the merge costs about one memory
// round trip next to the row plan and the rope angles.
constexpr int kMaxSplit = 64;
// MS: upper bound of the split count (registers per thread); EX: the count is
// exactly MS, so no per-split guard is needed
template <int D, int MS, bool EX>
__global__ __launch_bounds__(D / 2) void k_attn_combine(AttnArgs A) {
  const int rh = blockIdx.x;
  const int r = rh / A.H, h = rh % A.H;
  const int pr = threadIdx.x;
  const int ns = EX ? MS : A.nsplit;
  __shared__ float rc[32], rs[32];
  __shared__ float sm[kMaxSplit], sl[kMaxSplit];
  const int64_t q0 = (int64_t)r * ns * A.H + h;   // partial row of split s: q0 + s * H
  uint32_t ov[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s)
    if (EX || s < ns) ov[s] = reinterpret_cast<const uint32_t *>(A.part_o + (q0 + (int64_t)s * A.H) * D)[pr];
  if (pr < ns) {
    sm[pr] = A.part_ml[2 * (q0 + (int64_t)pr * A.H)];
    sl[pr] = A.part_ml[2 * (q0 + (int64_t)pr * A.H) + 1];
  }
  const float sg = A.sinks ? A.sinks[h] * kLog2e : -INFINITY;
  const int b = A.seq[r];
  const int64_t p = (A.pos0 ? A.pos0[b] : 0) + A.tok[r];
  const int R = A.rope_dim;
  if (pr < R / 2) rope_cs_f((double)p, A.inv_freq[pr], 1.f, &rc[pr], &rs[pr]);
  __syncthreads();
  float M = sg;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, sm[s]);
  float den = A.sinks ? exp2f(sg - M) : 0.f;
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    if (EX || s < ns) {
      const float ms = sm[s];
      // the split's weight: its sum at the common max (0 for a split without
      // rows, whose partial output is zero); the exponent is <= 0
      const float f = ms == -INFINITY ? 0.f : sl[s] * __builtin_amdgcn_exp2f(ms - M);
      den += f;
      _Float16 h0, h1;
      const uint16_t lo = (uint16_t)(ov[s] & 0xFFFFu), hi = (uint16_t)(ov[s] >> 16);
      __builtin_memcpy(&h0, &lo, 2);
      __builtin_memcpy(&h1, &hi, 2);
      o0 = fmaf((float)h0, f, o0);
      o1 = fmaf((float)h1, f, o1);
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  o0 *= inv;
  o1 *= inv;
  const int d0 = 2 * pr;
  if (d0 >= D - R) {
    const int pi = (d0 - (D - R)) >> 1;
    const float a = o0 * rc[pi] + o1 * rs[pi], bb = -o0 * rs[pi] + o1 * rc[pi];
    o0 = a;
    o1 = bb;
  }
  const int64_t oe = ((int64_t)r * A.H + h) * D + d0;
  if (A.out_dtype == DSV4_F32) *reinterpret_cast<float2 *>((float *)A.out + oe) = make_float2(o0, o1);
  else *reinterpret_cast<uint32_t *>((uint16_t *)A.out + oe) = pack_bf16x2(o0, o1);
}

// -------------------------------------------------------------------- fp32 path
// One workgroup (256 threads) per query row.  Requires H*D <= 8192, H <= 64,
// D <= 512, float32 rows and queries.
__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs A, int D) {
  extern __shared__ float sm[];
  const int H = A.H;
  float *qs = sm;                 // [H*D]
  float *rows = qs + H * D;       // [32*D]
  float *lg = rows + 32 * D;      // [H*32]
  float *mrun = lg + H * 32;      // [H]
  float *alph = mrun + H;         // [H]
  float *lrun = alph + H;         // [H]
  __shared__ int sel[kMaxSel];
  __shared__ float rc[32], rs[32];
  __shared__ int sh_cnt[kMaxSel / 64];
  const int tid = threadIdx.x;
  const int r = blockIdx.x;
  RowPlan P = row_plan(A, r);
  if (A.csa && A.topk > 0) P.nsel = compact_idx<256>(A, r, P.pcount, sel, sh_cnt, true);
  const int nrows = P.nwin + P.nsel;
  const int R = A.rope_dim;
  if (tid < R / 2) rope_cs_f((double)P.p, A.inv_freq[tid], 1.f, &rc[tid], &rs[tid]);
  __syncthreads();
  const float *q = (const float *)A.q + (int64_t)r * H * D;
  for (int e = tid; e < H * D / 2; e += 256) {
    const int hh = e / (D / 2), d0 = 2 * (e % (D / 2));
    float x0 = q[hh * D + d0], x1 = q[hh * D + d0 + 1];
    if (d0 >= D - R) {
      const int pi = (d0 - (D - R)) >> 1;
      const float a = x0 * rc[pi] - x1 * rs[pi], bb = x0 * rs[pi] + x1 * rc[pi];
      x0 = a;
      x1 = bb;
    }
    qs[hh * D + d0] = x0 * A.scale_log2;
    qs[hh * D + d0 + 1] = x1 * A.scale_log2;
  }
  for (int hh = tid; hh < H; hh += 256) { mrun[hh] = -INFINITY; lrun[hh] = 0.f; }
  constexpr int MAXO = 32;        // (H*D/2) / 256 pairs per thread at most
  float o0[MAXO], o1[MAXO];
#pragma unroll
  for (int u = 0; u < MAXO; ++u) { o0[u] = 0.f; o1[u] = 0.f; }
  const int npairs = H * D / 2;
  for (int base = 0; base < nrows; base += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * D; e += 256) {
      const int j = e / D, d = e % D;
      float v = 0.f;
      if (base + j < nrows) {
        float sc;
        const uint8_t *rp = row_ptr(A, P, sel, base + j, &sc);
        v = reinterpret_cast<const float *>(rp)[d];
      }
      rows[e] = v;
    }
    __syncthreads();
    for (int e = tid; e < H * 32; e += 256) {
      const int hh = e / 32, j = e % 32;
      float d = -INFINITY;
      if (base + j < nrows) {
        d = 0.f;
        for (int k = 0; k < D; ++k) d = fmaf(qs[hh * D + k], rows[j * D + k], d);
      }
      lg[e] = d;
    }
    __syncthreads();
    for (int hh = tid; hh < H; hh += 256) {
      float mx = mrun[hh];
      for (int j = 0; j < 32; ++j) mx = fmaxf(mx, lg[hh * 32 + j]);
      const float al = exp2f(mrun[hh] - mx);
      float sum = 0.f;
      for (int j = 0; j < 32; ++j) {
        const float pj = exp2f(lg[hh * 32 + j] - mx);
        lg[hh * 32 + j] = pj;
        sum += pj;
      }
      lrun[hh] = lrun[hh] * al + sum;
      mrun[hh] = mx;
      alph[hh] = al;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < MAXO; ++u) {
      const int e = tid + 256 * u;
      if (e < npairs) {
        const int hh = e / (D / 2), d0 = 2 * (e % (D / 2));
        const float al = alph[hh];
        float a0 = o0[u] * al, a1 = o1[u] * al;
        for (int j = 0; j < 32; ++j) {
          const float pj = lg[hh * 32 + j];
          a0 = fmaf(pj, rows[j * D + d0], a0);
          a1 = fmaf(pj, rows[j * D + d0 + 1], a1);
        }
        o0[u] = a0;
        o1[u] = a1;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < MAXO; ++u) {
    const int e = tid + 256 * u;
    if (e < npairs) {
      const int hh = e / (D / 2), d0 = 2 * (e % (D / 2));
      const float mr = mrun[hh];
      float f = 1.f, den = lrun[hh];
      if (A.sinks) {
        const float sg = A.sinks[hh] * kLog2e;
        const float M = fmaxf(mr, sg);
        f = exp2f(mr - M);
        den = lrun[hh] * f + exp2f(sg - M);
      }
      const float inv = den > 0.f ? f / den : 0.f;
      float x0 = o0[u] * inv, x1 = o1[u] * inv;
      if (d0 >= D - R) {
        const int pi = (d0 - (D - R)) >> 1;
        const float a = x0 * rc[pi] + x1 * rs[pi], bb = -x0 * rs[pi] + x1 * rc[pi];
        x0 = a;
        x1 = bb;
      }
      const int64_t oe = ((int64_t)r * H + hh) * D + d0;
      if (A.out_dtype == DSV4_F32) *reinterpret_cast<float2 *>((float *)A.out + oe) = make_float2(x0, x1);
      else *reinterpret_cast<uint32_t *>((uint16_t *)A.out + oe) = pack_bf16x2(x0, x1);
    }
  }
}

}  // namespace dsv4

using namespace dsv4;

namespace dsv4host {

static RowSrc mk_src(const dsv4_rows *rw) {
  RowSrc s{};
  if (!rw) return s;
  s.data = (const uint8_t *)rw->data;
  s.rscale = rw->row_scale;
  s.count = rw->count;
  s.first_tok = rw->first_tok;
  s.stride = rw->seq_stride;
  s.dtype = rw->dtype;
  s.tail = rw->tail;
  s.ring = rw->ring ? 1 : 0;
  switch (rw->dtype) {
  case DSV4_F32: s.rbytes = 4LL * rw->dim; break;
  case DSV4_BF16: s.rbytes = 2LL * rw->dim; break;
  case DSV4_F16: s.rbytes = 2LL * rw->dim; break;
  case DSV4_FP8R: s.rbytes = (int64_t)(rw->dim - rw->tail) + 2LL * rw->tail; break;
  default: s.rbytes = 0;
  }
  return s;
}

static std::atomic<int> g_batch_invariant{0};

int set_batch_invariant(bool on) { return g_batch_invariant.exchange(on ? 1 : 0); }

static std::atomic<int> g_diag_on{0};

int set_diagnostics(bool on) { return g_diag_on.exchange(on ? 1 : 0); }

// The current device's counters to out (after every queued kernel finished),
// cleared if reset.
int read_diagnostics(uint64_t *out, bool reset) {
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_diag), sizeof(uint64_t) * DSV4_DIAG_COUNT, 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess && reset) {
    static const uint64_t zero[DSV4_DIAG_COUNT] = {};
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_diag), zero, sizeof zero, 0, hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) return fail(DSV4_EHIP, "read_diagnostics: %s", hipGetErrorString(e));
  return DSV4_OK;
}

// Splits per query (decode): enough workgroups to occupy the chip, but at least
// four 32-row tiles per split, because every split writes a 64 x 512 fp16
// partial (normalised by its own sum) plus fp32 (max, sum) per head that the
// combine kernel reads back.
int attn_nsplit(int T, int64_t max_rows) {
  const int64_t tiles = (max_rows + 31) / 32;
  // batch-invariant mode: one workgroup reduces a query's rows in one order
  if (g_batch_invariant.load(std::memory_order_relaxed)) return 1;
  if (T < 1 || T >= 512 || tiles < 8) return 1;
  int64_t want = (256 + T - 1) / T;
  const int64_t cap = tiles / 4;
  if (want > cap) want = cap;
  if (want > 64) want = 64;
  return want < 1 ? 1 : (int)want;
}

size_t attn_ws(int T, int H, int D, int64_t max_rows) {
  const int ns = attn_nsplit(T, max_rows);
  if (ns <= 1) return 0;
  return (size_t)T * ns * H * ((size_t)D * 2 + 8) + 256;   // fp16 outputs, fp32 (max, sum)
}

// the merge kernel instance with the smallest split bound that holds nsplit
static void launch_combine(const AttnArgs &A, int T, int H, hipStream_t st) {
  const dim3 g((unsigned)((int64_t)T * H)), b(256);
  const int ns = A.nsplit;
  if (ns == 8) hipLaunchKernelGGL((k_attn_combine<512, 8, true>), g, b, 0, st, A);
  else if (ns < 8) hipLaunchKernelGGL((k_attn_combine<512, 8, false>), g, b, 0, st, A);
  else if (ns == 16) hipLaunchKernelGGL((k_attn_combine<512, 16, true>), g, b, 0, st, A);
  else if (ns < 16) hipLaunchKernelGGL((k_attn_combine<512, 16, false>), g, b, 0, st, A);
  else if (ns == 32) hipLaunchKernelGGL((k_attn_combine<512, 32, true>), g, b, 0, st, A);
  else if (ns < 32) hipLaunchKernelGGL((k_attn_combine<512, 32, false>), g, b, 0, st, A);
  else if (ns == kMaxSplit) hipLaunchKernelGGL((k_attn_combine<512, kMaxSplit, true>), g, b, 0, st, A);
  else hipLaunchKernelGGL((k_attn_combine<512, kMaxSplit, false>), g, b, 0, st, A);
}

int launch_attn(const dsv4_queries *q, const void *qv, int q_dtype, int H, int D, const dsv4_rows *win, int W,
                const dsv4_rows *pool, const int32_t *idx, int topk, int m, int csa, const float *sinks,
                float sm_scale, int rope_dim, double theta, void *out, int out_dtype, void *ws,
                int64_t max_rows, hipStream_t st) {
  const int T = q->n_rows;
  if (T == 0) return DSV4_OK;
  AttnArgs A{};
  A.seq = q->seq;
  A.tok = q->tok;
  A.pos0 = q->pos0;
  A.q = qv;
  A.T = T;
  A.H = H;
  A.qdtype = q_dtype;
  A.win = mk_src(W > 0 ? win : nullptr);
  A.W = W > 0 ? W : 0;
  A.pool = mk_src(pool);
  A.idx = idx;
  A.topk = csa ? topk : 0;
  A.m = m;
  A.csa = csa;
  A.sinks = sinks;
  A.scale_log2 = sm_scale * kLog2e;
  A.rope_dim = rope_dim;
  A.theta = theta;
  for (int i = 0; i < 32; ++i) A.inv_freq[i] = (i < rope_dim / 2) ? pow(theta, -2.0 * i / (double)rope_dim) : 0.0;
  A.out = out;
  A.out_dtype = out_dtype;
  A.diag = g_diag_on.load(std::memory_order_relaxed);
  if (q_dtype == DSV4_F32) {
    A.nsplit = 1;
    const size_t lds = ((size_t)H * D + 32 * (size_t)D + 32 * (size_t)H + 3 * (size_t)H) * 4;
    hipLaunchKernelGGL(k_attn_f32, dim3(T), dim3(256), lds, st, A, D);
    return check_launch("k_attn_f32");
  }
  const int ns = attn_nsplit(T, max_rows);
  A.nsplit = ns;
  if (ns > 1) {
    A.part_o = (uint16_t *)ws;
    A.part_ml = (float *)(A.part_o + (size_t)T * ns * H * D);
  }
  const bool fp8 = (W > 0 && win->dtype == DSV4_FP8R) || (pool && pool->dtype == DSV4_FP8R);
  const bool f16 = (W > 0 ? win->dtype == DSV4_F16 : true) && (pool ? pool->dtype == DSV4_F16 : true) &&
                   (W > 0 || pool);
  // FP8 rows in the 448 E4M3 + 64 bf16 layout take the DMA-staged path too
  const bool fp8fast = fp8 && D == 512 && (W > 0 ? win->tail == 64 : true) && (pool ? pool->tail == 64 : true);
  dim3 grid((unsigned)((int64_t)T * ns));
  if (fp8fast && (H == 16 || H == 32 || H == 64)) {
#define DSV4_DECK(NHB)                                                                              \
  if (rope_dim == 64) hipLaunchKernelGGL((k_attn_dec<NHB, true>), grid, dim3(NHB * 128), 0, st, A); \
  else hipLaunchKernelGGL((k_attn_dec<NHB, false>), grid, dim3(NHB * 128), 0, st, A);
    switch (H) {
    case 16: DSV4_DECK(1) break;
    case 32: DSV4_DECK(2) break;
    default: DSV4_DECK(4) break;
    }
#undef DSV4_DECK
    int rc = check_launch("k_attn_dec");
    if (rc || ns == 1) return rc;
    launch_combine(A, T, H, st);
    return check_launch("k_attn_combine");
  }
  if (f16 || fp8fast) {
#define DSV4_F16K(NW)                                                                                 \
  if (rope_dim == 64) hipLaunchKernelGGL((k_attn_f16<1, NW, false, true>), grid, dim3(NW * 64), 0, st, A); \
  else hipLaunchKernelGGL((k_attn_f16<1, NW, false, false>), grid, dim3(NW * 64), 0, st, A);
    if (fp8fast) {   // FP8 rows with 16, 32 or 64 heads took k_attn_dec above: 48 heads
      if (rope_dim == 64) hipLaunchKernelGGL((k_attn_f16<1, 3, true, true>), grid, dim3(3 * 64), 0, st, A);
      else hipLaunchKernelGGL((k_attn_f16<1, 3, true, false>), grid, dim3(3 * 64), 0, st, A);
    } else {
      switch (H) {
      case 16: DSV4_F16K(1) break;
      case 32: DSV4_F16K(2) break;
      case 48: DSV4_F16K(3) break;
      default: DSV4_F16K(4) break;
      }
    }
#undef DSV4_F16K
    int rc = check_launch("k_attn_f16");
    if (rc || ns == 1) return rc;
    launch_combine(A, T, H, st);
    return check_launch("k_attn_combine");
  }
  switch (H / 16) {
#define DSV4_ATT(NW)                                                                                  \
  case NW:                                                                                            \
    if (fp8) hipLaunchKernelGGL((k_attn_mfma<512, NW, true>), grid, dim3(NW * 64), 0, st, A);         \
    else hipLaunchKernelGGL((k_attn_mfma<512, NW, false>), grid, dim3(NW * 64), 0, st, A);            \
    break;
    DSV4_ATT(1)
    DSV4_ATT(2)
    DSV4_ATT(3)
    DSV4_ATT(4)
#undef DSV4_ATT
  }
  int rc = check_launch("k_attn_mfma");
  if (rc || ns == 1) return rc;
  launch_combine(A, T, H, st);
  return check_launch("k_attn_combine");
}

}  // namespace dsv4host
