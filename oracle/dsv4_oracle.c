/*
 * dsv4_oracle.c -- plain fp64 CPU oracle for the DeepSeek-V4 hybrid attention
 * path (Compressed Sparse Attention and Heavily Compressed Attention).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path
 * (the HIP library) never calls it and shares no code, header or table with it.
 *
 * Every step is written the slow, obvious way: fp64 scalar loops, no blocking,
 * no fusion, inputs decoded exactly from their storage type.  OpenMP only
 * splits independent query rows / entries across threads; it never changes the
 * order of any sum.
 *
 * Sources (the HF Transformers DeepSeek-V4 model page, "Hybrid attention" and
 * "Attention mask layout"; the jagaldol review, "CSA" / "HCA"; the insight.ai.kr
 * write-up; the MarkTechPost summary).  Where those pages leave a step open the
 * reading used here is stated beside the step.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

/* storage types understood by the oracle's own decoders */
enum { OR_F32 = 0, OR_BF16 = 1, OR_FP8R = 2, OR_MXFP4 = 3, OR_F64 = 4, OR_F16 = 5 };

/* A set of per-sequence rows (a compressed pool or a sliding window).
 * Row i of sequence b starts at byte (b*seq_stride + i) * row_bytes.
 * FP8R rows: (dim - tail) OCP e4m3 bytes followed by `tail` bf16 values,
 *            times one fp32 scale per row (row_scale[b*seq_stride+i]) that
 *            applies to the e4m3 part only.
 * MXFP4 rows: dim/2 bytes of E2M1 nibbles (low nibble = even element) and
 *            dim/32 E8M0 block scales in blk_scale[(b*seq_stride+i)*dim/32 ..].
 * count[b]     : number of valid rows of sequence b.
 * first_tok[b] : token index of row 0 (windows); NULL for pools.            */
typedef struct {
  const void *data;
  const float *row_scale;
  const uint8_t *blk_scale;
  int32_t dtype, dim, tail;
  int64_t seq_stride;
  const int32_t *count;
  const int32_t *first_tok;
} or_rows;

/* ------------------------------------------------------------------------ */
/* Storage decoders, from the published format definitions.                 */
/* ------------------------------------------------------------------------ */

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double or_bf16_to_f64(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 mantissa bits. */
double or_f16_to_f64(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double mag;
  if (e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
  if (e == 0) mag = ldexp((double)m, -24);
  else mag = ldexp(1.0 + (double)m / 1024.0, e - 15);
  return s ? -mag : mag;
}

/* OCP FP8 E4M3 ("fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits;
 * no infinities, S.1111.111 is NaN, largest finite magnitude 448. */
double or_e4m3_to_f64(uint8_t v) {
  int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) mag = ldexp((double)m / 8.0, -6);
  else mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* OCP MX E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit. */
double or_e2m1_to_f64(uint8_t nib) {
  int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
  double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -mag : mag;
}

/* OCP MX E8M0 shared scale: 2^(e-127); 0xFF is NaN. */
double or_e8m0_to_f64(uint8_t e) {
  if (e == 255) return NAN;
  return ldexp(1.0, (int)e - 127);
}

static int64_t row_bytes(const or_rows *r) {
  switch (r->dtype) {
  case OR_F32: return 4LL * r->dim;
  case OR_F64: return 8LL * r->dim;
  case OR_BF16: return 2LL * r->dim;
  case OR_F16: return 2LL * r->dim;
  case OR_FP8R: return (int64_t)(r->dim - r->tail) + 2LL * r->tail;
  case OR_MXFP4: return r->dim / 2;
  }
  return 0;
}

/* Decode one stored vector of `dim` elements into fp64.
 * `scale` is the FP8R row scale, `bs` the MXFP4 block scales. */
static void decode_vec(const uint8_t *p, int dtype, int dim, int tail, double scale,
                       const uint8_t *bs, double *out) {
  int d;
  switch (dtype) {
  case OR_F32:
    for (d = 0; d < dim; d++) { float f; memcpy(&f, p + 4 * d, 4); out[d] = f; }
    break;
  case OR_F64:
    for (d = 0; d < dim; d++) memcpy(&out[d], p + 8 * d, 8);
    break;
  case OR_BF16:
    for (d = 0; d < dim; d++) { uint16_t h; memcpy(&h, p + 2 * d, 2); out[d] = or_bf16_to_f64(h); }
    break;
  case OR_F16:
    for (d = 0; d < dim; d++) { uint16_t h; memcpy(&h, p + 2 * d, 2); out[d] = or_f16_to_f64(h); }
    break;
  case OR_FP8R:
    for (d = 0; d < dim - tail; d++) out[d] = or_e4m3_to_f64(p[d]) * scale;
    for (d = 0; d < tail; d++) {
      uint16_t h; memcpy(&h, p + (dim - tail) + 2 * d, 2);
      out[dim - tail + d] = or_bf16_to_f64(h);
    }
    break;
  case OR_MXFP4:
    for (d = 0; d < dim; d++) {
      uint8_t byte = p[d / 2];
      uint8_t nib = (d & 1) ? (byte >> 4) : (byte & 15);
      out[d] = or_e2m1_to_f64(nib) * or_e8m0_to_f64(bs[d / 32]);
    }
    break;
  }
}

static void decode_row(const or_rows *r, int b, int64_t i, double *out) {
  int64_t g = (int64_t)b * r->seq_stride + i;
  const uint8_t *p = (const uint8_t *)r->data + g * row_bytes(r);
  double sc = (r->dtype == OR_FP8R) ? (double)r->row_scale[g] : 1.0;
  const uint8_t *bs = (r->dtype == OR_MXFP4) ? r->blk_scale + g * (r->dim / 32) : NULL;
  decode_vec(p, r->dtype, r->dim, r->tail, sc, bs, out);
}

/* Exported for the codec tests: decode n vectors of `dim` elements. */
void or_decode(const void *data, int dtype, int64_t n, int dim, int tail,
               const float *row_scale, const uint8_t *blk_scale, double *out) {
  or_rows r;
  int64_t i;
  memset(&r, 0, sizeof r);
  r.data = data; r.dtype = dtype; r.dim = dim; r.tail = tail;
  r.row_scale = row_scale; r.blk_scale = blk_scale; r.seq_stride = n;
  for (i = 0; i < n; i++) decode_row(&r, 0, i, out + i * dim);
}

/* ------------------------------------------------------------------------ */
/* O1: partial RoPE, interleaved pairs on the last rope_dim channels.        */
/* HF DeepSeek-V4 page, "Hybrid attention", backbone bullet on partial RoPE: */
/* pairs (2i, 2i+1) of the trailing qk_rope_head_dim channels rotate; the    */
/* same rotation at position -p is applied to the output's rope slice.       */
/* Frequencies: f_i = theta^(-2i/R) (standard RoPE schedule; reading).       */
/* ------------------------------------------------------------------------ */
static void rope_vec(double *x, int dim, int R, double pos, double theta, int sign) {
  int i;
  for (i = 0; i < R / 2; i++) {
    double f = pow(theta, -2.0 * i / (double)R);
    double a = (double)sign * pos * f;
    double c = cos(a), s = sin(a);
    double *pr = x + (dim - R) + 2 * i;
    double x0 = pr[0], x1 = pr[1];
    pr[0] = x0 * c - x1 * s;
    pr[1] = x0 * s + x1 * c;
  }
}

void or_rope(double *x, int64_t n_rows, int dim, int rope_dim, const double *pos,
             double theta, int sign) {
  int64_t r;
#pragma omp parallel for schedule(static)
  for (r = 0; r < n_rows; r++) rope_vec(x + r * dim, dim, rope_dim, pos[r], theta, sign);
}

/* ------------------------------------------------------------------------ */
/* O2: KV compressor (softmax-gated pooling with a learned position bias).   */
/* HF page "Hybrid attention" (CSA: overlapping windows, m=4; HCA: non-      */
/* overlapping windows, m'=128); insight.ai.kr paragraph on CSA (softmax-    */
/* gated pooling, learned position bias); jagaldol "CSA" step 1.             */
/* Readings: the gate is per channel; CSA entry s pools tokens               */
/* [(s-1)m, (s+1)m) (window 2m, stride m, the previous block at local        */
/* offsets 0..m-1 and the current block at m..2m-1); HCA entry s pools       */
/* [s m, (s+1) m).  Tokens outside [0, S) do not take part.  N = floor(S/m). */
/* The KV stream is then rotated at P_s = pos0 + s*m.                        */
/* ------------------------------------------------------------------------ */
void or_compress(const void *c, const void *z, int in_dtype, const double *bias,
                 int B, int S, int dim, int m, int overlap, int rope_dim, double theta,
                 const int64_t *pos0, double *pool) {
  int N = S / m;
  int64_t task;
  int64_t elt = (in_dtype == OR_F32) ? 4 : (in_dtype == OR_F64 ? 8 : 2);
#pragma omp parallel for schedule(static)
  for (task = 0; task < (int64_t)B * N; task++) {
    int b = (int)(task / N), s = (int)(task % N);
    int t0 = overlap ? (s - 1) * m : s * m;   /* first token of the window */
    int width = overlap ? 2 * m : m;
    double *out = pool + task * dim;
    double *cv = (double *)malloc(sizeof(double) * dim);
    double *zv = (double *)malloc(sizeof(double) * dim);
    double *mx = (double *)malloc(sizeof(double) * dim);
    double *den = (double *)malloc(sizeof(double) * dim);
    int j, d;
    for (d = 0; d < dim; d++) { mx[d] = -INFINITY; den[d] = 0.0; out[d] = 0.0; }
    /* pass 1: per-channel max of the gate logits z + B over the window */
    for (j = 0; j < width; j++) {
      int t = t0 + j;
      if (t < 0 || t >= S) continue;
      decode_vec((const uint8_t *)z + ((int64_t)b * S + t) * dim * elt, in_dtype, dim, 0, 1.0, NULL, zv);
      for (d = 0; d < dim; d++) {
        double g = zv[d] + bias[(int64_t)j * dim + d];
        if (g > mx[d]) mx[d] = g;
      }
    }
    /* pass 2: softmax weights and the weighted sum of the candidates c */
    for (j = 0; j < width; j++) {
      int t = t0 + j;
      if (t < 0 || t >= S) continue;
      decode_vec((const uint8_t *)z + ((int64_t)b * S + t) * dim * elt, in_dtype, dim, 0, 1.0, NULL, zv);
      decode_vec((const uint8_t *)c + ((int64_t)b * S + t) * dim * elt, in_dtype, dim, 0, 1.0, NULL, cv);
      for (d = 0; d < dim; d++) {
        double e = exp(zv[d] + bias[(int64_t)j * dim + d] - mx[d]);
        den[d] += e;
        out[d] += e * cv[d];
      }
    }
    for (d = 0; d < dim; d++) out[d] /= den[d];
    if (rope_dim > 0) {
      double P = (double)((pos0 ? pos0[b] : 0) + (int64_t)s * m);
      rope_vec(out, dim, rope_dim, P, theta, +1);
    }
    free(cv); free(zv); free(mx); free(den);
  }
}

/* O3: visibility.  Entry w of a pool with stride m is visible to query token */
/* t iff its source window has closed: w < floor((t+1)/m) (HF page, "Attention */
/* mask layout", HCA paragraph), capped by the number of stored entries.      */
static int64_t n_visible(int64_t t, int m, int64_t count) {
  int64_t n = (t + 1) / m;
  return n < count ? n : count;
}

/* ------------------------------------------------------------------------ */
/* O4: Lightning Indexer scores.                                              */
/* insight.ai.kr: ReLU-scored multi-head dot products, FP4 on the q/k path;   */
/* HF page: the indexer scores each query against the compressed pool.       */
/* Reading: I(t,s) = scale * sum_h w[t,h] * max(0, q_I[t,h] . k_I[s]).        */
/* scores[q, s] for s < n(t); every other slot is set to -inf.                */
/* q_I rows are [n_q, H, Di] in q_dtype (F32 / BF16 / MXFP4 with block scales */
/* q_scale [n_q, H, Di/32]).                                                  */
/* ------------------------------------------------------------------------ */
void or_index_scores(int n_q, const int32_t *q_seq, const int32_t *q_tok, const void *q_idx,
                     const uint8_t *q_scale, int q_dtype, const double *w, int H, int Di,
                     const or_rows *kpool, int m, double scale, double *scores, int nmax) {
  int qi;
  int64_t qrow = (q_dtype == OR_MXFP4) ? Di / 2 : (int64_t)Di * (q_dtype == OR_F32 ? 4 : (q_dtype == OR_F64 ? 8 : 2));
#pragma omp parallel for schedule(dynamic, 1)
  for (qi = 0; qi < n_q; qi++) {
    int b = q_seq[qi];
    int64_t n = n_visible(q_tok[qi], m, kpool->count[b]);
    double *qv = (double *)malloc(sizeof(double) * (size_t)H * Di);
    double *kv = (double *)malloc(sizeof(double) * Di);
    int h, d;
    int64_t s;
    for (h = 0; h < H; h++) {
      int64_t g = (int64_t)qi * H + h;
      decode_vec((const uint8_t *)q_idx + g * qrow, q_dtype, Di, 0, 1.0,
                 q_scale ? q_scale + g * (Di / 32) : NULL, qv + (int64_t)h * Di);
    }
    for (s = 0; s < nmax; s++) scores[(int64_t)qi * nmax + s] = -INFINITY;
    for (s = 0; s < n && s < nmax; s++) {
      double acc = 0.0;
      decode_row(kpool, b, s, kv);
      for (h = 0; h < H; h++) {
        double dot = 0.0;
        for (d = 0; d < Di; d++) dot += qv[(int64_t)h * Di + d] * kv[d];
        acc += w[(int64_t)qi * H + h] * (dot > 0.0 ? dot : 0.0);
      }
      scores[(int64_t)qi * nmax + s] = scale * acc;
    }
    free(qv); free(kv);
  }
}

/* ------------------------------------------------------------------------ */
/* O5: per-query top-k with the -1 sentinel.                                  */
/* HF page "Attention mask layout", CSA paragraph: each query keeps the top   */
/* index_topk blocks; queries before the first window closes get nothing and  */
/* the indexer's -1 sentinel propagates.  jagaldol "CSA" step 3.              */
/* Readings: candidates are s < n(t); larger score first, equal scores go to  */
/* the lower entry index; min(k, n) indices are written in ascending index    */
/* order, the remaining slots hold -1.                                        */
/* ------------------------------------------------------------------------ */
void or_topk(int n_q, const double *scores, int nmax, const int32_t *n_valid, int k,
             int32_t *idx_out) {
  int qi;
#pragma omp parallel for schedule(dynamic, 4)
  for (qi = 0; qi < n_q; qi++) {
    const double *sc = scores + (int64_t)qi * nmax;
    int n = n_valid[qi] < nmax ? n_valid[qi] : nmax;
    int take = k < n ? k : n;
    char *chosen = (char *)calloc((size_t)(n > 0 ? n : 1), 1);
    int r, s, o = 0;
    /* repeated selection of the best remaining candidate (slow, obvious) */
    for (r = 0; r < take; r++) {
      int best = -1;
      for (s = 0; s < n; s++) {
        if (chosen[s]) continue;
        if (best < 0 || sc[s] > sc[best]) best = s;   /* strict: ties keep the lower s */
      }
      chosen[best] = 1;
    }
    for (s = 0; s < n; s++)
      if (chosen[s]) idx_out[(int64_t)qi * k + o++] = s;
    for (; o < k; o++) idx_out[(int64_t)qi * k + o] = -1;
    free(chosen);
  }
}

/* ------------------------------------------------------------------------ */
/* O6 / O7: core attention with one shared K=V head.                          */
/* HF page "Hybrid attention" backbone: shared K=V multi-query attention      */
/* (num_key_value_heads = 1, the same tensor read as key and value); partial  */
/* RoPE on q and the inverse rotation (position -p) on the output rope slice; */
/* a learnable per-head sink; the sliding-window K=V branch concatenated with */
/* the compressor's entries.  "Attention mask layout": CSA queries see their  */
/* indexer picks only (-1 masked), HCA queries every entry w < (t+1)//m.      */
/* Readings: window = tokens [t-W+1, t] (W tokens including the query); the   */
/* sink is one extra logit with a zero value; logits are scaled by sm_scale;  */
/* window and pool rows are taken as stored (already rotated).                */
/* mode 0 (CSA): pool rows are idx[q, 0..k), -1 skipped.                      */
/* mode 1 (HCA): pool rows are every s < min(count, (t+1)//m).                */
/* out is [n_q, H, D] fp64.                                                   */
/* ------------------------------------------------------------------------ */
void or_attn(int n_q, const int32_t *q_seq, const int32_t *q_tok, const int64_t *pos0,
             const void *q, int q_dtype, int H, int D, const or_rows *win, int W,
             const or_rows *pool, int mode, const int32_t *idx, int k, int m,
             const double *sinks, double sm_scale, int rope_dim, double theta, double *out) {
  int qi;
  int64_t qelt = (q_dtype == OR_F32) ? 4 : (q_dtype == OR_F64 ? 8 : 2);
#pragma omp parallel for schedule(dynamic, 1)
  for (qi = 0; qi < n_q; qi++) {
    int b = q_seq[qi];
    int64_t t = q_tok[qi];
    double p = (double)((pos0 ? pos0[b] : 0) + t);
    int64_t nrows_max = (int64_t)(W > 0 ? W : 0) + (mode == 0 ? k : (pool ? pool->count[b] : 0));
    double *rows = (double *)malloc(sizeof(double) * (size_t)(nrows_max > 0 ? nrows_max : 1) * D);
    double *qv = (double *)malloc(sizeof(double) * D);
    double *lg = (double *)malloc(sizeof(double) * (size_t)(nrows_max > 0 ? nrows_max : 1));
    int64_t nr = 0, j, s;
    int h, d, i;
    /* gather the key/value rows of this query */
    if (W > 0 && win) {
      int64_t ft = win->first_tok ? win->first_tok[b] : 0;
      int64_t lo = t - W + 1;
      if (lo < ft) lo = ft;
      if (lo < 0) lo = 0;
      for (j = lo; j <= t && j - ft < win->count[b]; j++) decode_row(win, b, j - ft, rows + (nr++) * D);
    }
    if (pool) {
      if (mode == 0) {
        for (i = 0; i < k; i++) {
          s = idx[(int64_t)qi * k + i];
          if (s < 0) continue;
          decode_row(pool, b, s, rows + (nr++) * D);
        }
      } else {
        int64_t n = n_visible(t, m, pool->count[b]);
        for (s = 0; s < n; s++) decode_row(pool, b, s, rows + (nr++) * D);
      }
    }
    for (h = 0; h < H; h++) {
      double mx, den, *o = out + ((int64_t)qi * H + h) * D;
      int64_t g = (int64_t)qi * H + h;
      decode_vec((const uint8_t *)q + g * D * qelt, q_dtype, D, 0, 1.0, NULL, qv);
      if (rope_dim > 0) rope_vec(qv, D, rope_dim, p, theta, +1);
      mx = sinks ? sinks[h] : -INFINITY;
      for (j = 0; j < nr; j++) {
        double acc = 0.0;
        for (d = 0; d < D; d++) acc += qv[d] * rows[j * D + d];
        lg[j] = acc * sm_scale;
        if (lg[j] > mx) mx = lg[j];
      }
      den = sinks ? exp(sinks[h] - mx) : 0.0;   /* the sink adds to the denominator only */
      for (d = 0; d < D; d++) o[d] = 0.0;
      for (j = 0; j < nr; j++) {
        double e = exp(lg[j] - mx);
        den += e;
        for (d = 0; d < D; d++) o[d] += e * rows[j * D + d];
      }
      for (d = 0; d < D; d++) o[d] = (den > 0.0) ? o[d] / den : 0.0;
      if (rope_dim > 0) rope_vec(o, D, rope_dim, p, theta, -1);
    }
    free(rows); free(qv); free(lg);
  }
}

/* ------------------------------------------------------------------------ */
/* Q1/Q2: storage encoders for quantise-on-write (insight.ai.kr deep dive:  */
/* the KV cache is FP8 with the RoPE channels kept in BF16; MarkTechPost:    */
/* the indexer's query/key path is MXFP4).  The pages give the formats, not  */
/* the scale recipe; the readings here: FP8 rows take one fp32 scale         */
/* s = amax/448 over the E4M3 channels (s = 1 for an all-zero row), codes    */
/* are the E4M3 value nearest to x/s (ties to the even code, the sign of     */
/* x/s kept, 448 at most); MXFP4 blocks of 32 take the OCP MX scale          */
/* 2^(floor(log2 amax) - 2) (2^-127 for an all-zero block, exponent clamped  */
/* to [-127, 127]), codes are the E2M1 value nearest to x/scale, saturated   */
/* at 6, ties to the even code, no negative zero.  The scale and x/s are     */
/* formed in fp32, the precision the GPU kernel decides them in; the nearest */
/* code is then found by searching every code of the format.                 */
/* ------------------------------------------------------------------------ */
static uint8_t nearest_e4m3(float v) {
  const int neg = signbit(v) ? 1 : 0;
  double best = INFINITY;
  int c, code = 0;
  for (c = 0; c < 127; c++) {   /* magnitudes 0x00..0x7E (0x7F is NaN) */
    const double d = fabs(fabs((double)v) - or_e4m3_to_f64((uint8_t)c));
    if (d < best || (d == best && (c & 1) == 0)) {
      best = d;
      code = c;
    }
  }
  return (uint8_t)(code | (neg << 7));
}

static uint8_t nearest_e2m1(double v) {
  const double a = fabs(v) > 6.0 ? 6.0 : fabs(v);
  double best = INFINITY;
  int c, code = 0;
  for (c = 0; c < 8; c++) {
    const double d = fabs(a - or_e2m1_to_f64((uint8_t)c));
    if (d < best || (d == best && (c & 1) == 0)) {
      best = d;
      code = c;
    }
  }
  if (code != 0 && v < 0) code |= 8;
  return (uint8_t)code;
}

/* x: n rows of dim fp32 values.  rows: n x ((dim - tail) + 2 tail) bytes;
 * scales: n fp32. */
void or_quantize_fp8r(int64_t n, int dim, int tail, const float *x, uint8_t *rows, float *scales) {
  int64_t i;
  const int64_t rb = (int64_t)(dim - tail) + 2LL * tail;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; i++) {
    const float *xr = x + i * dim;
    uint8_t *o = rows + i * rb;
    float amax = 0.f, s;
    int d;
    for (d = 0; d < dim - tail; d++)
      if (fabsf(xr[d]) > amax) amax = fabsf(xr[d]);
    s = amax > 0.f ? amax / 448.0f : 1.0f;
    scales[i] = s;
    for (d = 0; d < dim - tail; d++) o[d] = nearest_e4m3(xr[d] / s);
    for (d = 0; d < tail; d++) {   /* bf16: the nearer of the two neighbours, ties to even */
      const double v = (double)xr[dim - tail + d];
      uint32_t u;
      uint16_t lo, hi, h;
      memcpy(&u, &xr[dim - tail + d], 4);
      lo = (uint16_t)(u >> 16);   /* truncation: same sign, magnitude just below (or equal) */
      hi = (uint16_t)(lo + 1);
      {
        const double dl = fabs(v - or_bf16_to_f64(lo)), dh = fabs(v - or_bf16_to_f64(hi));
        h = (dl < dh || (dl == dh && (lo & 1) == 0)) ? lo : hi;
      }
      memcpy(o + (dim - tail) + 2 * d, &h, 2);
    }
  }
}

/* x: n rows of dim fp32 values (dim a multiple of 32).  rows: n x dim/2 bytes
 * (low nibble = even element); scales: n x dim/32 E8M0 bytes. */
void or_quantize_mxfp4(int64_t n, int dim, const float *x, uint8_t *rows, uint8_t *scales) {
  int64_t i;
#pragma omp parallel for schedule(static)
  for (i = 0; i < n; i++) {
    int blk, d;
    for (blk = 0; blk < dim / 32; blk++) {
      const float *xb = x + i * dim + 32 * blk;
      float amax = 0.f;
      int e;
      for (d = 0; d < 32; d++)
        if (fabsf(xb[d]) > amax) amax = fabsf(xb[d]);
      if (amax > 0.f) {
        int k;
        frexp((double)amax, &k);   /* amax = f 2^k, f in [0.5, 1): floor(log2 amax) = k - 1 */
        e = k - 1 - 2;
        if (e < -127) e = -127;
        if (e > 127) e = 127;
      } else {
        e = -127;
      }
      scales[i * (dim / 32) + blk] = (uint8_t)(e + 127);
      for (d = 0; d < 32; d += 2) {
        const uint8_t lo = nearest_e2m1(ldexp((double)xb[d], -e));
        const uint8_t hi = nearest_e2m1(ldexp((double)xb[d + 1], -e));
        rows[i * (dim / 2) + 16 * blk + d / 2] = (uint8_t)(lo | (hi << 4));
      }
    }
  }
}

int or_num_threads(void) { return omp_get_max_threads(); }
void or_set_num_threads(int n) { omp_set_num_threads(n); }
