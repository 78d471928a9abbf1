// dsv4_api.cpp -- the C ABI of libdsv4: host-side argument validation, kernel
// selection and error reporting.  Every check runs before anything is queued,
// so a failing call launches nothing.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime.h>

#include "dsv4.h"

namespace dsv4host {

static thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSV4_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DSV4_OK;
}

// launchers (defined next to their kernels)
int launch_compress(const void *c, const void *z, int in_dtype, const float *bias, int B, int S, int dim, int m,
                    int overlap, int rope_dim, double theta, const int64_t *pos0, void *pool, int out_dtype,
                    hipStream_t st);
int launch_rope(const void *x, int x_dtype, void *y, int y_dtype, int64_t n_rows, int dim, int rope_dim,
                const int64_t *pos, double theta, int inverse, hipStream_t st);
size_t index_topk_ws(int64_t n_rows, int64_t stride, int topk);
size_t index_topk_scratch_bytes();
int index_topk_scratch(void **ptr);
int index_topk_supported(int64_t stride, int topk);
int launch_index_topk(const dsv4_queries *q, const void *qv, const uint8_t *qscale, int q_dtype, const float *w,
                      int H, int Di, const dsv4_rows *kp, int m, int topk, float scale, int32_t *idx_out,
                      float *score_out, void *ws, hipStream_t st);
int attn_nsplit(int T, int64_t max_rows);
size_t attn_ws(int T, int H, int D, int64_t max_rows);
int set_batch_invariant(bool on);
int set_diagnostics(bool on);
int read_diagnostics(uint64_t *out, bool reset);
int launch_cache_append(const dsv4_cache *C, int n, const int32_t *n_new, const void *kv, const void *kv_c,
                        const void *kv_z, const void *idx_c, const void *idx_z, int in_dtype, hipStream_t st);
int launch_linear(const void *x, int64_t ldx, const void *w, int64_t ldw, void *y, int64_t ldy, int y_dtype, int M,
                  int N, int K, int groups, int64_t gx, int64_t gw, int64_t gy, hipStream_t st);
int launch_quantize(const void *x, int x_dtype, int64_t n, int dim, int tail, void *rows, float *row_scale,
                    uint8_t *blk_scale, int out_dtype, hipStream_t st);
int launch_attn(const dsv4_queries *q, const void *qv, int q_dtype, int H, int D, const dsv4_rows *win, int W,
                const dsv4_rows *pool, const int32_t *idx, int topk, int m, int csa, const float *sinks,
                float sm_scale, int rope_dim, double theta, void *out, int out_dtype, void *ws, int64_t max_rows,
                hipStream_t st);

// a stored-row format of the cache writer: dtype, dim and tail
static int check_store(const char *what, int dtype, int dim, int tail, const void *rsc, const void *bsc, bool mx_ok) {
  if (dim < 64 || dim > 512 || dim % 64) return fail(DSV4_ENOTSUP, "%s: dim %d (64..512, multiple of 64)", what, dim);
  switch (dtype) {
  case DSV4_F32:
  case DSV4_BF16:
  case DSV4_F16:
    if (tail != 0) return fail(DSV4_EINVAL, "%s: tail %d without FP8R", what, tail);
    return DSV4_OK;
  case DSV4_FP8R:
    if (!rsc) return fail(DSV4_EINVAL, "%s: FP8R rows need row scales", what);
    if (tail < 0 || tail >= dim || tail % 8) return fail(DSV4_ENOTSUP, "%s: FP8R tail %d (multiple of 8, < dim)", what, tail);
    return DSV4_OK;
  case DSV4_MXFP4:
    if (!mx_ok) return fail(DSV4_ENOTSUP, "%s: MXFP4 is a pool format only", what);
    if (!bsc) return fail(DSV4_EINVAL, "%s: MXFP4 rows need block scales", what);
    if (tail != 0) return fail(DSV4_EINVAL, "%s: MXFP4 takes no tail", what);
    return DSV4_OK;
  }
  return fail(DSV4_EINVAL, "%s: unknown dtype %d", what, dtype);
}

static int check_stream(const char *what, const dsv4_stream *s, const void *c, const void *z) {
  int rc = check_store(what, s->pool_dtype, s->dim, s->tail, s->row_scale, s->blk_scale, true);
  if (rc) return rc;
  if (!s->pos_bias || !s->buf || !s->pool || !s->count || s->pool_cap < 0)
    return fail(DSV4_EINVAL, "%s: NULL pos_bias/buf/pool/count or negative pool_cap", what);
  if (s->rope_dim < 0 || (s->rope_dim & 1) || s->rope_dim > 64)
    return fail(DSV4_EINVAL, "%s: rope_dim %d (even, <= 64)", what, s->rope_dim);
  if (!c || !z) return fail(DSV4_EINVAL, "%s: NULL inputs c/z", what);
  return DSV4_OK;
}

static int ok() {
  g_err[0] = 0;
  return DSV4_OK;
}

static int check_queries(const dsv4_queries *q) {
  if (!q) return fail(DSV4_EINVAL, "queries: NULL descriptor");
  if (q->n_rows < 0 || q->n_seq < 1) return fail(DSV4_EINVAL, "queries: n_rows %d, n_seq %d", q->n_rows, q->n_seq);
  if (q->n_rows > 0 && (!q->seq || !q->tok)) return fail(DSV4_EINVAL, "queries: seq/tok arrays are NULL");
  return DSV4_OK;
}

static int check_rows(const dsv4_rows *r, const char *what, int dim) {
  if (!r) return fail(DSV4_EINVAL, "%s: NULL descriptor", what);
  if ((!r->data && r->seq_stride > 0) || !r->count) return fail(DSV4_EINVAL, "%s: data/count is NULL", what);
  if (r->dim != dim) return fail(DSV4_EINVAL, "%s: dim %d, expected %d", what, r->dim, dim);
  if (r->seq_stride < 0) return fail(DSV4_EINVAL, "%s: negative seq_stride", what);
  if (r->ring && (!r->first_tok || r->seq_stride < 1))
    return fail(DSV4_EINVAL, "%s: the ring layout is for windows (first_tok set, seq_stride >= 1)", what);
  if (r->dtype == DSV4_FP8R) {
    if (!r->row_scale && r->seq_stride > 0) return fail(DSV4_EINVAL, "%s: FP8R rows need row_scale", what);
    if (r->tail < 0 || r->tail > dim || (r->tail % 8) != 0 || ((dim - r->tail) % 8) != 0)
      return fail(DSV4_ENOTSUP, "%s: FP8R tail %d (multiple of 8 within dim required)", what, r->tail);
  } else if (r->dtype == DSV4_MXFP4) {
    if (!r->blk_scale && r->seq_stride > 0) return fail(DSV4_EINVAL, "%s: MXFP4 rows need blk_scale", what);
  } else if (r->dtype != DSV4_F32 && r->dtype != DSV4_BF16 && r->dtype != DSV4_F16) {
    return fail(DSV4_EINVAL, "%s: unknown dtype %d", what, r->dtype);
  }
  return DSV4_OK;
}

}  // namespace dsv4host

using namespace dsv4host;

extern "C" {

const char *dsv4_last_error(void) { return g_err; }

const char *dsv4_version(void) { return "dsv4-gfx950 0.1"; }

int dsv4_quantize(const void *x, int32_t x_dtype, int64_t n_rows, int32_t dim, int32_t tail, void *rows_out,
                  float *row_scale_out, uint8_t *blk_scale_out, int32_t out_dtype, hipStream_t stream) {
  if (n_rows < 0) return fail(DSV4_EINVAL, "quantize: n_rows %lld", (long long)n_rows);
  if (x_dtype != DSV4_F32 && x_dtype != DSV4_BF16 && x_dtype != DSV4_F16)
    return fail(DSV4_ENOTSUP, "quantize: input dtype %d", x_dtype);
  if (dim < 64 || dim > 512 || dim % 64) return fail(DSV4_ENOTSUP, "quantize: dim %d (64..512, multiple of 64)", dim);
  if (out_dtype == DSV4_FP8R) {
    if (tail < 0 || tail >= dim || (tail & 1)) return fail(DSV4_EINVAL, "quantize: tail %d", tail);
    if (n_rows > 0 && (!x || !rows_out || !row_scale_out)) return fail(DSV4_EINVAL, "quantize: NULL x/rows/row_scale");
  } else if (out_dtype == DSV4_MXFP4) {
    if (tail != 0) return fail(DSV4_EINVAL, "quantize: MXFP4 takes no bf16 tail (tail %d)", tail);
    if (n_rows > 0 && (!x || !rows_out || !blk_scale_out)) return fail(DSV4_EINVAL, "quantize: NULL x/rows/blk_scale");
  } else {
    return fail(DSV4_ENOTSUP, "quantize: output dtype %d (FP8R or MXFP4)", out_dtype);
  }
  const int rc = launch_quantize(x, x_dtype, n_rows, dim, tail, rows_out, row_scale_out, blk_scale_out, out_dtype,
                                 stream);
  return rc ? rc : ok();
}

int dsv4_cache_append(const dsv4_cache *C, int32_t n, const int32_t *n_new, const void *kv, const void *kv_c,
                      const void *kv_z, const void *idx_c, const void *idx_z, int32_t in_dtype, hipStream_t stream) {
  if (!C) return fail(DSV4_EINVAL, "cache_append: NULL cache");
  if (C->n_seq < 1 || C->n_seq > 65535 || n < 0)
    return fail(DSV4_EINVAL, "cache_append: n_seq %d (1..65535), n %d", C->n_seq, n);
  if (C->m < 1 || C->m > 1024) return fail(DSV4_ENOTSUP, "cache_append: m %d (1..1024)", C->m);
  if (!C->len) return fail(DSV4_EINVAL, "cache_append: NULL len");
  if (in_dtype != DSV4_F32 && in_dtype != DSV4_BF16) return fail(DSV4_ENOTSUP, "cache_append: input dtype %d", in_dtype);
  int rc = check_stream("cache_append: kv stream", &C->kv, kv_c, kv_z);
  if (rc) return rc;
  if (C->idx.dim != 0 && (rc = check_stream("cache_append: idx stream", &C->idx, idx_c, idx_z))) return rc;
  if (C->win_cap < 0) return fail(DSV4_EINVAL, "cache_append: win_cap %d", C->win_cap);
  if (C->win_cap > 0) {
    if ((rc = check_store("cache_append: window", C->win_dtype, C->win_dim, C->win_tail, C->win_scale, nullptr, false)))
      return rc;
    if (C->win_dim != C->kv.dim) return fail(DSV4_EINVAL, "cache_append: win_dim %d != kv dim %d", C->win_dim, C->kv.dim);
    if (!C->win || !C->win_count || !C->win_first || !kv)
      return fail(DSV4_EINVAL, "cache_append: NULL window rows/count/first or kv input");
    if (C->win_rope_dim < 0 || (C->win_rope_dim & 1) || C->win_rope_dim > 64)
      return fail(DSV4_EINVAL, "cache_append: win_rope_dim %d (even, <= 64)", C->win_rope_dim);
  }
  const bool rot = C->kv.rope_dim > 0 || C->idx.rope_dim > 0 || (C->win_cap > 0 && C->win_rope_dim > 0);
  if (rot && !(C->rope_theta > 0)) return fail(DSV4_EINVAL, "cache_append: rope_theta must be > 0");
  const int64_t items = (C->win_cap > 0 ? (int64_t)(n < C->win_cap ? n : C->win_cap) : 0) +
                        (C->idx.dim ? 2 : 1) * (((int64_t)n + C->m - 1) / C->m);
  if (items > 0x7fffffff) return fail(DSV4_ENOTSUP, "cache_append: n %d too large for one append", n);
  rc = launch_cache_append(C, n, n_new, kv, kv_c, kv_z, idx_c, idx_z, in_dtype, stream);
  return rc ? rc : ok();
}

int dsv4_linear(const void *x, int64_t ldx, const void *w, int64_t ldw, void *y, int64_t ldy, int32_t y_dtype,
                int32_t M, int32_t N, int32_t K, int32_t groups, int64_t x_group_stride, int64_t w_group_stride,
                int64_t y_group_stride, hipStream_t stream) {
  if (M < 0 || N < 0 || K < 0 || groups < 0) return fail(DSV4_EINVAL, "linear: M %d N %d K %d groups %d", M, N, K, groups);
  if (M == 0 || N == 0 || groups == 0) return ok();
  if (!x || !w || !y) return fail(DSV4_EINVAL, "linear: NULL x/w/y");
  if (K == 0 || K % 64) return fail(DSV4_ENOTSUP, "linear: K %d (a positive multiple of 64)", K);
  if (y_dtype != DSV4_F32 && y_dtype != DSV4_BF16 && y_dtype != DSV4_F16)
    return fail(DSV4_ENOTSUP, "linear: output dtype %d (F32, BF16 or F16)", y_dtype);
  if (ldx < K || ldw < K || ldy < N || ldx % 8 || ldw % 8)
    return fail(DSV4_EINVAL, "linear: row strides x %lld w %lld (>= K, multiples of 8) y %lld (>= N)", (long long)ldx,
                (long long)ldw, (long long)ldy);
  if ((x_group_stride | w_group_stride) % 8 || (((uintptr_t)x | (uintptr_t)w) & 15))
    return fail(DSV4_EINVAL, "linear: x and w must be 16-byte aligned with group strides that keep them so");
  if (M > 65535 * 128 || groups > 65535) return fail(DSV4_ENOTSUP, "linear: M %d / groups %d too large", M, groups);
  const int rc = launch_linear(x, ldx, w, ldw, y, ldy, y_dtype, M, N, K, groups, x_group_stride, w_group_stride,
                               y_group_stride, stream);
  return rc ? rc : ok();
}

int dsv4_set_batch_invariant(int32_t on) { return dsv4host::set_batch_invariant(on != 0); }

int dsv4_set_diagnostics(int32_t on) { return dsv4host::set_diagnostics(on != 0); }

int dsv4_read_diagnostics(uint64_t *out, int32_t reset) {
  if (!out) return fail(DSV4_EINVAL, "read_diagnostics: NULL output");
  const int rc = dsv4host::read_diagnostics(out, reset != 0);
  return rc ? rc : ok();
}

int dsv4_compress(const void *c, const void *z, int32_t in_dtype, const float *pos_bias, int32_t n_seq,
                  int32_t seq_len, int32_t dim, int32_t m, int32_t overlap, int32_t rope_dim, double rope_theta,
                  const int64_t *pos0, void *pool, int32_t out_dtype, hipStream_t stream) {
  if (n_seq < 0 || seq_len < 0 || m < 1) return fail(DSV4_EINVAL, "compress: n_seq %d seq_len %d m %d", n_seq, seq_len, m);
  if (n_seq > 65535) return fail(DSV4_ENOTSUP, "compress: n_seq %d (at most 65535)", n_seq);
  const bool empty = n_seq == 0 || seq_len / m == 0;   // nothing to pool: pointers may be NULL
  if (!empty && (!c || !z || !pos_bias || !pool)) return fail(DSV4_EINVAL, "compress: NULL tensor pointer");
  if (dim < 2 || (dim & 1) || dim > 4096) return fail(DSV4_ENOTSUP, "compress: dim %d (even, 2..4096)", dim);
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > dim || rope_dim > 64)
    return fail(DSV4_EINVAL, "compress: rope_dim %d (even, <= min(dim, 64))", rope_dim);
  if ((in_dtype != DSV4_F32 && in_dtype != DSV4_BF16) ||
      (out_dtype != DSV4_F32 && out_dtype != DSV4_BF16 && out_dtype != DSV4_F16))
    return fail(DSV4_ENOTSUP, "compress: dtypes in %d (F32/BF16) out %d (F32/BF16/F16)", in_dtype, out_dtype);
  if (rope_dim > 0 && !(rope_theta > 0)) return fail(DSV4_EINVAL, "compress: rope_theta must be > 0");
  const int rc = launch_compress(c, z, in_dtype, pos_bias, n_seq, seq_len, dim, m, overlap ? 1 : 0, rope_dim,
                                 rope_theta, pos0, pool, out_dtype, stream);
  return rc ? rc : ok();
}

int dsv4_rope(const void *x, int32_t x_dtype, void *y, int32_t y_dtype, int64_t n_rows, int32_t dim,
              int32_t rope_dim, const int64_t *pos, double rope_theta, int32_t inverse, hipStream_t stream) {
  if (n_rows > 0 && (!x || !y || !pos)) return fail(DSV4_EINVAL, "rope: NULL pointer");   // no rows: may be NULL
  if (n_rows < 0) return fail(DSV4_EINVAL, "rope: n_rows %lld", (long long)n_rows);
  if (dim < 2 || (dim & 1) || dim > 4096) return fail(DSV4_ENOTSUP, "rope: dim %d (even, 2..4096)", dim);
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > dim || rope_dim > 64)
    return fail(DSV4_EINVAL, "rope: rope_dim %d (even, <= min(dim, 64))", rope_dim);
  if ((x_dtype != DSV4_F32 && x_dtype != DSV4_BF16) ||
      (y_dtype != DSV4_F32 && y_dtype != DSV4_BF16 && y_dtype != DSV4_F16))
    return fail(DSV4_ENOTSUP, "rope: dtypes x %d (F32/BF16) y %d (F32/BF16/F16)", x_dtype, y_dtype);
  if (x == y && x_dtype != y_dtype) return fail(DSV4_EINVAL, "rope: in-place needs equal dtypes");
  if (rope_dim > 0 && !(rope_theta > 0)) return fail(DSV4_EINVAL, "rope: rope_theta must be > 0");
  const int rc = launch_rope(x, x_dtype, y, y_dtype, n_rows, dim, rope_dim, pos, rope_theta, inverse, stream);
  return rc ? rc : ok();
}

size_t dsv4_index_topk_workspace(int32_t n_rows, int64_t pool_seq_stride, int32_t topk) {
  if (n_rows < 0 || pool_seq_stride < 0 || topk < 1) return 0;
  return index_topk_ws(n_rows, pool_seq_stride, topk);
}

// Argument checks shared by dsv4_index_topk and dsv4_index_topk_noalloc;
// *need receives the scratch bytes the call uses.
static int index_topk_check(const dsv4_queries *q, const void *q_idx, const uint8_t *q_idx_scale, int32_t q_dtype,
                            const float *w, int32_t n_heads, int32_t head_dim, const dsv4_rows *k_pool, int32_t m,
                            int32_t topk, float score_scale, int32_t *idx_out, size_t *need) {
  int rc = check_queries(q);
  if (rc) return rc;
  if (q->n_rows > 0 && (!q_idx || !w || !idx_out)) return fail(DSV4_EINVAL, "index_topk: NULL tensor pointer");
  if (m < 1 || topk < 1 || topk > 2048) return fail(DSV4_EINVAL, "index_topk: m %d topk %d (1..2048)", m, topk);
  if ((rc = check_rows(k_pool, "index_topk: k_pool", head_dim))) return rc;
  if (k_pool->ring) return fail(DSV4_EINVAL, "index_topk: k_pool cannot be a ring");
  if (k_pool->dtype != q_dtype) return fail(DSV4_ENOTSUP, "index_topk: key dtype %d != query dtype %d", k_pool->dtype, q_dtype);
  if (!(score_scale > 0)) return fail(DSV4_EINVAL, "index_topk: score_scale must be > 0");
  if (q_dtype == DSV4_F32) {
    if (n_heads < 1 || head_dim < 1 || (size_t)(n_heads * head_dim + n_heads) * 4 > 65536)
      return fail(DSV4_ENOTSUP, "index_topk: fp32 path needs n_heads*head_dim <= 16000 (%d x %d)", n_heads, head_dim);
  } else if (q_dtype == DSV4_BF16) {
    if (n_heads < 16 || n_heads > 64 || n_heads % 16 || head_dim < 32 || head_dim > 128 || head_dim % 32)
      return fail(DSV4_ENOTSUP, "index_topk: bf16 path needs n_heads in {16,32,48,64}, head_dim in {32,64,96,128} (%d, %d)",
                  n_heads, head_dim);
  } else if (q_dtype == DSV4_MXFP4) {
    if (n_heads < 16 || n_heads > 64 || n_heads % 16 || head_dim != 128)
      return fail(DSV4_ENOTSUP, "index_topk: MXFP4 path needs n_heads in {16,32,48,64} and head_dim 128 (%d, %d)",
                  n_heads, head_dim);
    if (q->n_rows > 0 && !q_idx_scale) return fail(DSV4_EINVAL, "index_topk: MXFP4 queries need q_idx_scale");
  } else {
    return fail(DSV4_ENOTSUP, "index_topk: query dtype %d", q_dtype);
  }
  if (!index_topk_supported(k_pool->seq_stride, topk))
    return fail(DSV4_ENOTSUP, "index_topk: pool stride %lld (at most 65535 * 1024 entries)",
                (long long)k_pool->seq_stride);
  *need = index_topk_ws(q->n_rows, k_pool->seq_stride, topk);
  return DSV4_OK;
}

int dsv4_index_topk(const dsv4_queries *q, const void *q_idx, const uint8_t *q_idx_scale, int32_t q_dtype,
                    const float *w, int32_t n_heads, int32_t head_dim, const dsv4_rows *k_pool, int32_t m,
                    int32_t topk, float score_scale, int32_t *idx_out, float *score_out, void *ws, size_t ws_bytes,
                    hipStream_t stream) {
  size_t need = 0;
  int rc = index_topk_check(q, q_idx, q_idx_scale, q_dtype, w, n_heads, head_dim, k_pool, m, topk, score_scale,
                            idx_out, &need);
  if (rc) return rc;
  if (q->n_rows > 0 && (!ws || ws_bytes < need))
    return fail(DSV4_EWORKSPACE, "index_topk: workspace %zu bytes, need %zu", ws_bytes, need);
  rc = launch_index_topk(q, q_idx, q_idx_scale, q_dtype, w, n_heads, head_dim, k_pool, m, topk, score_scale, idx_out,
                         score_out, ws, stream);
  return rc ? rc : ok();
}

int dsv4_index_topk_noalloc(const dsv4_queries *q, const void *q_idx, const uint8_t *q_idx_scale, int32_t q_dtype,
                            const float *w, int32_t n_heads, int32_t head_dim, const dsv4_rows *k_pool, int32_t m,
                            int32_t topk, float score_scale, int32_t *idx_out, float *score_out, hipStream_t stream) {
  size_t need = 0;
  int rc = index_topk_check(q, q_idx, q_idx_scale, q_dtype, w, n_heads, head_dim, k_pool, m, topk, score_scale,
                            idx_out, &need);
  if (rc) return rc;
  if (need > index_topk_scratch_bytes())
    return fail(DSV4_EWORKSPACE, "index_topk_noalloc: the call needs %zu scratch bytes, the static scratch holds %zu",
                need, index_topk_scratch_bytes());
  if (q->n_rows == 0) return ok();
  void *scr = nullptr;
  if ((rc = index_topk_scratch(&scr))) return rc;
  rc = launch_index_topk(q, q_idx, q_idx_scale, q_dtype, w, n_heads, head_dim, k_pool, m, topk, score_scale, idx_out,
                         score_out, scr, stream);
  return rc ? rc : ok();
}

size_t dsv4_attn_workspace(int32_t n_rows, int32_t n_heads, int32_t dim, int64_t max_rows_per_query) {
  if (n_rows < 0 || n_heads < 1 || dim < 1 || max_rows_per_query < 0) return 0;
  return attn_ws(n_rows, n_heads, dim, max_rows_per_query);
}

static int attn_common(const char *who, const dsv4_queries *q, const void *qv, int32_t q_dtype, int32_t n_heads,
                       int32_t dim, const dsv4_rows *window, int32_t W, const dsv4_rows *pool, int pool_needed,
                       int32_t rope_dim, double rope_theta, void *out, int32_t out_dtype) {
  int rc = check_queries(q);
  if (rc) return rc;
  if (q->n_rows > 0 && (!qv || !out)) return fail(DSV4_EINVAL, "%s: NULL q/out", who);   // no rows: may be NULL
  if (W < 0) return fail(DSV4_EINVAL, "%s: W %d", who, W);
  if (W > 0 && (rc = check_rows(window, "window", dim))) return rc;
  if (W > 0 && !window->first_tok) return fail(DSV4_EINVAL, "%s: window rows need first_tok", who);
  if (pool_needed && (rc = check_rows(pool, "pool", dim))) return rc;
  if (pool_needed && pool->ring) return fail(DSV4_EINVAL, "%s: a pool cannot be a ring", who);
  if (rope_dim < 0 || (rope_dim & 1) || rope_dim > dim || rope_dim > 64)
    return fail(DSV4_EINVAL, "%s: rope_dim %d (even, <= min(dim, 64))", who, rope_dim);
  if (rope_dim > 0 && !(rope_theta > 0)) return fail(DSV4_EINVAL, "%s: rope_theta must be > 0", who);
  if (out_dtype != DSV4_F32 && out_dtype != DSV4_BF16) return fail(DSV4_ENOTSUP, "%s: out dtype %d", who, out_dtype);
  const int wdt = W > 0 ? window->dtype : -1, pdt = pool_needed ? pool->dtype : -1;
  if (q_dtype == DSV4_F32) {
    if ((W > 0 && wdt != DSV4_F32) || (pool_needed && pdt != DSV4_F32))
      return fail(DSV4_ENOTSUP, "%s: fp32 queries need fp32 rows", who);
    if (n_heads < 1 || n_heads > 64 || dim < 2 || dim > 512 || (dim & 1) || n_heads * dim > 16384 ||
        ((size_t)n_heads * dim + 32 * (size_t)dim + 35 * (size_t)n_heads) * 4 > 65536)
      return fail(DSV4_ENOTSUP, "%s: fp32 path limits (n_heads %d, dim %d)", who, n_heads, dim);
  } else if (q_dtype == DSV4_BF16) {
    if (dim != 512) return fail(DSV4_ENOTSUP, "%s: bf16 path needs dim 512 (got %d)", who, dim);
    if (n_heads < 16 || n_heads > 64 || n_heads % 16)
      return fail(DSV4_ENOTSUP, "%s: bf16 path needs n_heads in {16,32,48,64} (got %d)", who, n_heads);
    const bool ok_w = W == 0 || wdt == DSV4_BF16 || wdt == DSV4_FP8R || wdt == DSV4_F16;
    const bool ok_p = !pool_needed || pdt == DSV4_BF16 || pdt == DSV4_FP8R || pdt == DSV4_F16;
    if (!ok_w || !ok_p) return fail(DSV4_ENOTSUP, "%s: bf16 queries need F16, BF16 or FP8R rows", who);
    if (W > 0 && pool_needed && wdt != pdt) return fail(DSV4_ENOTSUP, "%s: window and pool dtypes differ", who);
  } else {
    return fail(DSV4_ENOTSUP, "%s: query dtype %d", who, q_dtype);
  }
  return DSV4_OK;
}

int dsv4_sparse_attn(const dsv4_queries *q, const void *qv, int32_t q_dtype, int32_t n_heads, int32_t dim,
                     const dsv4_rows *window, int32_t W, const dsv4_rows *pool, const int32_t *idx, int32_t topk,
                     const float *sinks, float sm_scale, int32_t rope_dim, double rope_theta, void *out,
                     int32_t out_dtype, void *ws, size_t ws_bytes, hipStream_t stream) {
  if (topk < 0 || topk > 2048) return fail(DSV4_EINVAL, "sparse_attn: topk %d (0..2048)", topk);
  int rc = attn_common("sparse_attn", q, qv, q_dtype, n_heads, dim, window, W, pool, topk > 0, rope_dim, rope_theta,
                       out, out_dtype);
  if (rc) return rc;
  if (q->n_rows > 0 && topk > 0 && !idx) return fail(DSV4_EINVAL, "sparse_attn: idx is NULL");
  const int64_t max_rows = (int64_t)W + topk;
  const size_t need = attn_ws(q->n_rows, n_heads, dim, max_rows);
  if (q_dtype != DSV4_F32 && need > 0 && (!ws || ws_bytes < need))
    return fail(DSV4_EWORKSPACE, "sparse_attn: workspace %zu bytes, need %zu", ws_bytes, need);
  rc = launch_attn(q, qv, q_dtype, n_heads, dim, window, W, topk > 0 ? pool : nullptr, idx, topk, 1, 1, sinks,
                   sm_scale, rope_dim, rope_theta, out, out_dtype, ws, max_rows, stream);
  return rc ? rc : ok();
}

int dsv4_hca_attn(const dsv4_queries *q, const void *qv, int32_t q_dtype, int32_t n_heads, int32_t dim,
                  const dsv4_rows *window, int32_t W, const dsv4_rows *pool, int32_t m, const float *sinks,
                  float sm_scale, int32_t rope_dim, double rope_theta, void *out, int32_t out_dtype, void *ws,
                  size_t ws_bytes, hipStream_t stream) {
  if (m < 1) return fail(DSV4_EINVAL, "hca_attn: m %d", m);
  const int have_pool = pool != nullptr;
  int rc = attn_common("hca_attn", q, qv, q_dtype, n_heads, dim, window, W, pool, have_pool, rope_dim, rope_theta,
                       out, out_dtype);
  if (rc) return rc;
  const int64_t max_rows = (int64_t)W + (have_pool ? pool->seq_stride : 0);
  const size_t need = attn_ws(q->n_rows, n_heads, dim, max_rows);
  if (q_dtype != DSV4_F32 && need > 0 && (!ws || ws_bytes < need))
    return fail(DSV4_EWORKSPACE, "hca_attn: workspace %zu bytes, need %zu", ws_bytes, need);
  rc = launch_attn(q, qv, q_dtype, n_heads, dim, window, W, have_pool ? pool : nullptr, nullptr, 0, m, 0, sinks,
                   sm_scale, rope_dim, rope_theta, out, out_dtype, ws, max_rows, stream);
  return rc ? rc : ok();
}

}  // extern "C"
