/*
 * dsv4.h -- C ABI of the MI355X (gfx950) DeepSeek-V4 hybrid-attention hot path:
 * the KV compressor, the Lightning Indexer with top-k, Compressed Sparse
 * Attention (CSA) and Heavily Compressed Attention (HCA).
 *
 * Sources: the Hugging Face Transformers DeepSeek-V4 model page ("Hybrid
 * attention", "Attention mask layout", "Cache layers"); the jagaldol.com review
 * of the V4 paper ("CSA", "HCA"); the insight.ai.kr write-up of the HF blog
 * (pooling, indexer, storage precisions); the llm-atlas DeepSeek-V4-Flash card
 * (config.json fields); the MarkTechPost summary (MXFP4 indexer path).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major and
 *     contiguous as described per argument.  The library allocates nothing,
 *     keeps no pointer after the call returns (apart from work already queued)
 *     and holds no global state beyond its code objects, a thread-local error
 *     string, the batch-invariant and diagnostics switches, the per-GPU
 *     diagnostic counters and the static scratch array of
 *     dsv4_index_topk_noalloc (with its per-device address).
 *   - Every call validates its arguments on the host first; a call that returns
 *     an error has launched nothing.  dsv4_last_error() describes the failure.
 *   - The host checks pointers, sizes and formats, not the contents of device
 *     arrays (seq, tok, pos0, count, first_tok, picks): a pick outside
 *     [0, count[b]) is a masked row (-1 is the sentinel; the diagnostics count
 *     the others), and every other value must lie in its documented range, or
 *     the kernels may read outside the caller's buffers.
 *   - A call with nothing to do (no query rows, no rows to rotate or quantise,
 *     no entry to pool, an empty product) queues nothing and returns DSV4_OK;
 *     its tensor pointers may then be NULL (the row descriptors and scalar
 *     arguments are still checked).
 *   - Work is queued on `stream` (a hipStream_t; 0 = the null stream) with no
 *     host synchronisation.  A kernel fault surfaces at the caller's next
 *     synchronisation, or as DSV4_EHIP from a later call.
 *   - Positions: token t of sequence b has absolute position pos0[b] + t.
 *     pos0 may be NULL (all zero).
 */
#ifndef DSV4_H
#define DSV4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define DSV4_OK 0
#define DSV4_EINVAL (-1)     /* bad pointer, size or combination of arguments */
#define DSV4_ENOTSUP (-2)    /* valid but unsupported shape / dtype combination */
#define DSV4_EHIP (-3)       /* a HIP runtime call failed (launch error, earlier fault) */
#define DSV4_EWORKSPACE (-4) /* workspace pointer NULL or smaller than required */

/* ---- storage types ----
 * DSV4_F32   : float32.
 * DSV4_BF16  : bfloat16 (stored as 16-bit patterns).
 * DSV4_FP8R  : a K=V row of `dim` channels stored as (dim - tail) OCP FP8 E4M3
 *              bytes followed by `tail` bfloat16 values (the rope channels), plus
 *              one float32 scale per row applied to the E4M3 part (the FP8 KV,
 *              BF16 rope-dimension layout the insight.ai.kr write-up describes).
 *              Row size (dim - tail) + 2*tail bytes (576 for 512/64).
 * DSV4_MXFP4 : OCP MXFP4: E2M1 nibbles, low nibble = even element, dim/2 bytes
 *              per row, with one E8M0 scale byte per 32-element block in a
 *              separate plane (the MXFP4 indexer path of the MarkTechPost
 *              summary).
 * DSV4_F16   : IEEE binary16.  Offered as an output of the compressor and of
 *              the rope kernel so that prefill K=V rows can be staged straight
 *              into LDS for the fp16 matrix-core path; values must stay below
 *              65504 in magnitude. */
#define DSV4_F32 0
#define DSV4_BF16 1
#define DSV4_FP8R 2
#define DSV4_MXFP4 3
#define DSV4_F16 4

/* Query rows of one call: row r belongs to sequence seq[r] and is token tok[r]
 * (0-based) of that sequence.  Prefill: every token of every sequence; decode:
 * one row per sequence with tok = L_b - 1.  All arrays are device memory. */
typedef struct {
  int32_t n_rows;       /* T >= 0 */
  int32_t n_seq;        /* B >= 1 */
  const int32_t *seq;   /* [T], values in [0, B) */
  const int32_t *tok;   /* [T], values >= 0 */
  const int64_t *pos0;  /* [B] or NULL */
} dsv4_queries;

/* Per-sequence stored rows: a compressed pool or a sliding window.
 * Row i of sequence b lives at data + (b*seq_stride + i) * row_bytes(dtype).
 * count[b] rows are valid.  For a window, the valid rows hold the tokens
 * [first_tok[b], first_tok[b] + count[b]): token j is row j - first_tok[b]
 * (ring = 0), or row j mod seq_stride (ring = 1: the sliding-window ring that
 * dsv4_cache_append maintains).  For a pool, first_tok is NULL, ring is 0 and
 * row s is compressed entry s. */
typedef struct {
  const void *data;
  const float *row_scale;    /* DSV4_FP8R: [B*seq_stride]; else NULL */
  const uint8_t *blk_scale;  /* DSV4_MXFP4: [B*seq_stride, dim/32]; else NULL */
  int32_t dtype;
  int32_t dim;
  int32_t tail;              /* DSV4_FP8R: trailing bf16 channels; else 0 */
  int64_t seq_stride;        /* rows reserved per sequence (>= every count[b]) */
  const int32_t *count;      /* [B] */
  const int32_t *first_tok;  /* [B] (windows) or NULL (pools) */
  int32_t ring;              /* windows: 1 = ring layout (see above); pools: 0 */
} dsv4_rows;

/* dsv4_compress -- softmax-gated pooling with a learned position bias.
 * HF DeepSeek-V4 page, "Hybrid attention": CSA pools with overlapping windows
 * (compress_rate_csa m = 4), HCA with non-overlapping windows (m' = 128);
 * insight.ai.kr: softmax-gated pooling with a learned per-position bias.
 * Entry s, per channel d: weights softmax_t(z[t,d] + pos_bias[j(t),d]) over its
 * window, pooled[s,d] = sum_t weight * c[t,d].  overlap = 1: window
 * [(s-1)m, (s+1)m) with j = t - (s-1)m; overlap = 0: window [s m, (s+1)m) with
 * j = t - s m; tokens outside [0, seq_len) take no part.  Then, if rope_dim > 0,
 * the last rope_dim channels are rotated (interleaved pairs, frequencies
 * rope_theta^(-2i/rope_dim)) at position pos0[b] + s*m.
 *   c, z     : [n_seq, seq_len, dim], in_dtype DSV4_F32 or DSV4_BF16
 *   pos_bias : [2m or m, dim] float32
 *   pool     : [n_seq, seq_len / m, dim], out_dtype DSV4_F32, DSV4_BF16 or DSV4_F16
 * Partial trailing windows are not pooled.  dim even, <= 4096; n_seq <= 65535. */
int dsv4_compress(const void *c, const void *z, int32_t in_dtype, const float *pos_bias,
                  int32_t n_seq, int32_t seq_len, int32_t dim, int32_t m, int32_t overlap,
                  int32_t rope_dim, double rope_theta, const int64_t *pos0, void *pool,
                  int32_t out_dtype, hipStream_t stream);

/* dsv4_rope -- partial interleaved RoPE (HF page, "Hybrid attention", partial
 * RoPE bullet): for i < rope_dim/2 the channel pair (dim-R+2i, dim-R+2i+1) of
 * row r turns by angle sign * pos[r] * rope_theta^(-2i/R), sign = -1 when
 * inverse != 0.  Other channels are copied.  x: [n_rows, dim] in x_dtype
 * (DSV4_F32 or DSV4_BF16); y: [n_rows, dim] in y_dtype (DSV4_F32, DSV4_BF16 or
 * DSV4_F16); y may equal x when the dtypes match.  pos: [n_rows] int64 device. */
int dsv4_rope(const void *x, int32_t x_dtype, void *y, int32_t y_dtype, int64_t n_rows,
              int32_t dim, int32_t rope_dim, const int64_t *pos, double rope_theta,
              int32_t inverse, hipStream_t stream);

/* dsv4_index_topk -- Lightning Indexer scores and per-query top-k.
 * HF page "Hybrid attention" (the indexer scores queries against the pool and
 * keeps the top index_topk blocks) and "Attention mask layout" (-1 sentinel
 * before the first window closes); insight.ai.kr (ReLU-scored multi-head dot
 * products).  For query row r (sequence b, token t) and visible entry
 * s < n = min(k_pool->count[b], (t+1)/m):
 *     I(r,s) = score_scale * sum_h w[r,h] * max(0, q_idx[r,h,:] . k_pool[b,s,:])
 * idx_out[r, 0..min(topk,n)) receives the indices of the min(topk, n) largest
 * scores (equal scores: lower index first) in ascending index order; the rest
 * of the row is -1.  Scores are accumulated in fp32.
 *   q_idx       : [T, n_heads, head_dim] in q_dtype (DSV4_BF16, or DSV4_MXFP4 as
 *                 [T, n_heads, head_dim/2] bytes with q_idx_scale
 *                 [T, n_heads, head_dim/32] E8M0)
 *   w           : [T, n_heads] float32
 *   k_pool      : dtype equal to q_dtype, dim == head_dim
 *   idx_out     : [T, topk] int32
 *   score_out   : [T, topk] float32 scores of the picks (or -inf), may be NULL
 *   ws          : scratch of at least dsv4_index_topk_workspace(...) bytes
 * Supported: head_dim 128 (bf16: multiple of 32), n_heads multiple of 16 and
 * <= 64, 1 <= topk <= 2048, m >= 1, pool_seq_stride <= 65535 * 1024. */
size_t dsv4_index_topk_workspace(int32_t n_rows, int64_t pool_seq_stride, int32_t topk);
int dsv4_index_topk(const dsv4_queries *q, const void *q_idx, const uint8_t *q_idx_scale,
                    int32_t q_dtype, const float *w, int32_t n_heads, int32_t head_dim,
                    const dsv4_rows *k_pool, int32_t m, int32_t topk, float score_scale,
                    int32_t *idx_out, float *score_out, void *ws, size_t ws_bytes,
                    hipStream_t stream);

/* dsv4_index_topk_noalloc -- dsv4_index_topk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation and kernels, with the
 * workspace in a static scratch array of DSV4_NOALLOC_SCRATCH_BYTES inside
 * the library instead of a caller buffer.  Each GPU holds its own copy from
 * its first call until the process ends; every call on one GPU shares it, so
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be ordered by the caller.  The call allocates nothing; it returns
 * DSV4_EWORKSPACE (launching nothing) when
 * dsv4_index_topk_workspace(n_rows, pool_seq_stride, topk) exceeds the
 * scratch size (e.g. 32 decode rows over 32768-entry pools take 4 MiB, 8 rows
 * over 262144 entries 8 MiB).  Arguments and errors otherwise as
 * dsv4_index_topk. */
#define DSV4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int dsv4_index_topk_noalloc(const dsv4_queries *q, const void *q_idx, const uint8_t *q_idx_scale,
                            int32_t q_dtype, const float *w, int32_t n_heads, int32_t head_dim,
                            const dsv4_rows *k_pool, int32_t m, int32_t topk, float score_scale,
                            int32_t *idx_out, float *score_out, hipStream_t stream);

/* dsv4_sparse_attn -- CSA core attention (HF page, "Hybrid attention" backbone
 * bullets and "Attention mask layout", CSA paragraph).  One shared K=V head:
 * for query row r (sequence b, token t, position p = pos0[b] + t) and head h,
 * the key/value rows are the window rows holding tokens [t-W+1, t] and the pool
 * entries idx[r, 0..topk) that are not -1.  With q~ = RoPE(q[r,h], p):
 *     l_x = sm_scale * (q~ . x),  M = max(sinks[h], max_x l_x)
 *     o   = sum_x e^(l_x - M) x / (e^(sinks[h] - M) + sum_x e^(l_x - M))
 * and the last rope_dim channels of o are rotated back by -p.  Window and pool
 * rows are read as stored (already rotated).
 *   q      : [T, n_heads, dim] in q_dtype (DSV4_BF16 or DSV4_F32)
 *   window : W > 0 -> rows holding tokens (DSV4_F16 / DSV4_BF16 / DSV4_FP8R for
 *            bf16 queries, DSV4_F32 for fp32 queries);
 *            W = 0 -> no window branch (window may be NULL)
 *   pool   : same dtype as window, dim equal; may be NULL when topk = 0
 *   idx    : [T, topk] int32 in [-1, pool->count[b]); topk = 0: no pool branch
 *   sinks  : [n_heads] float32 or NULL (no sink)
 *   out    : [T, n_heads, dim] in out_dtype (DSV4_BF16 or DSV4_F32)
 *   ws     : scratch of at least dsv4_attn_workspace(...) bytes (may be 0 bytes)
 * A query with no rows and no sink gets a zero output.
 * Supported: bf16 queries -- dim 512, n_heads in {16, 32, 48, 64}, window and
 * pool rows DSV4_F16, DSV4_BF16 or DSV4_FP8R (one dtype for both); fp32
 * queries -- fp32 rows, any even dim <= 512 with 1..64 heads such that
 * n_heads*dim + 32*dim + 35*n_heads <= 16384; rope_dim even and <= 64,
 * topk <= 2048.
 * Range: the bf16 path runs its products on the fp16 matrix cores.  Stored
 * rows (DSV4_BF16 values, decoded DSV4_FP8R values) and the rotated queries
 * scaled by sm_scale*log2(e) must stay below 65504 in magnitude (larger values
 * become infinite and the output NaN); values below 2^-14 lose significand
 * bits to fp16's subnormal range (at most 2^-24 absolute).  Every workload
 * here is far inside that range (activations of a few units, FP8 rows at
 * most 448 x their row scale). */
size_t dsv4_attn_workspace(int32_t n_rows, int32_t n_heads, int32_t dim, int64_t max_rows_per_query);
int dsv4_sparse_attn(const dsv4_queries *q, const void *qv, int32_t q_dtype, int32_t n_heads,
                     int32_t dim, const dsv4_rows *window, int32_t W, const dsv4_rows *pool,
                     const int32_t *idx, int32_t topk, const float *sinks, float sm_scale,
                     int32_t rope_dim, double rope_theta, void *out, int32_t out_dtype,
                     void *ws, size_t ws_bytes, hipStream_t stream);

/* dsv4_hca_attn -- HCA core attention (HF page "Hybrid attention", HCA bullet:
 * no indexer, every pooled entry contributes; "Attention mask layout", HCA
 * paragraph: entry w is visible to token t iff w < (t+1)/m).  As
 * dsv4_sparse_attn with the pool rows s < min(pool->count[b], (t+1)/m) in place
 * of the idx set. */
int dsv4_hca_attn(const dsv4_queries *q, const void *qv, int32_t q_dtype, int32_t n_heads,
                  int32_t dim, const dsv4_rows *window, int32_t W, const dsv4_rows *pool,
                  int32_t m, const float *sinks, float sm_scale, int32_t rope_dim,
                  double rope_theta, void *out, int32_t out_dtype, void *ws, size_t ws_bytes,
                  hipStream_t stream);

/* dsv4_quantize -- quantise rows for storage (quantise-on-write of the decode
 * caches).  insight.ai.kr deep dive: the KV cache is FP8 with the RoPE
 * channels in BF16; MarkTechPost summary: the indexer's query/key path is
 * MXFP4.  Scale recipes (the pages give only the formats):
 *   DSV4_FP8R : per row s = amax/448 over channels [0, dim-tail) (1 for an
 *               all-zero row), code = E4M3 value nearest to x/s (ties to even,
 *               saturated at 448); channels [dim-tail, dim) as bf16 (round to
 *               nearest even).  rows_out [n_rows, (dim-tail) + 2*tail] bytes,
 *               row_scale_out [n_rows] float32.
 *   DSV4_MXFP4: per 32-channel block scale 2^(floor(log2 amax) - 2) (2^-127 for
 *               an all-zero block) as E8M0, code = E2M1 value nearest to
 *               x/scale (ties to even, saturated at 6, no negative zero).
 *               rows_out [n_rows, dim/2] bytes (low nibble = even channel),
 *               blk_scale_out [n_rows, dim/32]; tail must be 0.
 *   x : [n_rows, dim] in x_dtype (DSV4_F32, DSV4_BF16 or DSV4_F16), device.
 * Supported: dim a multiple of 64, at most 512; 0 <= tail < dim, tail even. */
int dsv4_quantize(const void *x, int32_t x_dtype, int64_t n_rows, int32_t dim, int32_t tail,
                  void *rows_out, float *row_scale_out, uint8_t *blk_scale_out, int32_t out_dtype,
                  hipStream_t stream);

/* dsv4_set_batch_invariant -- fixed reduction order across batch compositions
 * (DeepSeek-V4 review page, "Muon and MoE system": a token's result must be
 * bitwise the same whatever batch it is computed in).  on = 1: every query row
 * of the attention calls is reduced by one workgroup in one fixed order (no
 * split over its rows, whose count would depend on the batch size), so its
 * output does not depend on the other rows of the call.  The indexer scores,
 * top-k, compressor and rope are batch-invariant in either mode (one fixed
 * per-entry order; the choice among scoring kernels does not change it).
 * Process-wide; affects calls (and dsv4_attn_workspace sizes) made after it.
 * Returns the previous setting. */
int dsv4_set_batch_invariant(int32_t on);

/* dsv4_set_diagnostics / dsv4_read_diagnostics -- a debugging aid, off by
 * default.  While on, the attention calls (dsv4_sparse_attn, dsv4_hca_attn)
 * count into process-wide counters held on each GPU:
 *   DSV4_DIAG_REF_RAISES -- times a block of 16 heads raised its fixed
 *       softmax reference inside a tile because a logit passed it by more than
 *       2^15: the block's references become their heads' largest logits seen,
 *       the partial sums and accumulators scale by the power of two between
 *       the two references and the tile's probabilities are taken with the new
 *       ones (the result is the same either way; the count measures the extra
 *       work, about one softmax of the block per raise).  The prefill kernels
 *       raise each wave's 16 heads on their own; the FP8 decode kernel raises
 *       every head of a workgroup together and counts each block;
 *   DSV4_DIAG_BAD_PICKS -- idx entries that are neither the -1 sentinel nor a
 *       pool entry below the sequence's count (HF DeepSeek-V4 page, "Attention
 *       mask layout": only -1 marks an unused slot); attention treats such an
 *       entry like -1, and this counter is how a caller finds them.
 * Each pick entry is counted once per call whatever the split of its query.
 * Counting adds no work per row: the checks already run, and a workgroup adds
 * to a counter only when it has something to add.  Concurrent calls on one GPU
 * add to the same counters.  dsv4_set_diagnostics affects calls made after it
 * and returns the previous setting.  dsv4_read_diagnostics waits for the
 * current device's queued work, copies its DSV4_DIAG_COUNT counters to out
 * (host memory) and clears them if reset != 0; returns DSV4_OK or DSV4_EHIP. */
#define DSV4_DIAG_REF_RAISES 0
#define DSV4_DIAG_BAD_PICKS 1
#define DSV4_DIAG_COUNT 4
int dsv4_set_diagnostics(int32_t on);
int dsv4_read_diagnostics(uint64_t *out, int32_t reset);

/* ---- decode caches: streaming maintenance ----
 * HF DeepSeek-V4 page, "Cache layers": every compressed-attention layer carries
 * its compressor (and indexer) state from one forward call to the next -- a
 * sliding window of K=V rows plus, per compressed stream, a buffer of the
 * newest tokens, the pool and its count, with overlap state for CSA; the HCA
 * cache has one stream, the CSA cache a second one for the indexer keys at
 * index_head_dim.  insight.ai.kr deep dive: the KV cache is stored as FP8 with
 * the rope channels in BF16; MarkTechPost summary: MXFP4 indexer keys.
 *
 * One compressed stream.  The buffer keeps the candidates c and gates z of the
 * newest `span` tokens (span = 2m with overlap, else m): token t at slot
 * t mod span, as float32 [B, span, 2, dim] (c then z).  An entry is pooled,
 * rotated (rope_dim > 0) and quantised into the pool when its window closes. */
typedef struct {
  int32_t dim;               /* channels: multiple of 64, 64..512 */
  int32_t rope_dim;          /* trailing channels rotated at the entry position (0: none) */
  const float *pos_bias;     /* [span, dim] float32 */
  float *buf;                /* [B, span, 2, dim] float32 state */
  void *pool;                /* [B, pool_cap] rows of pool_dtype */
  float *row_scale;          /* DSV4_FP8R: [B, pool_cap]; else NULL */
  uint8_t *blk_scale;        /* DSV4_MXFP4: [B, pool_cap, dim/32]; else NULL */
  int32_t pool_dtype;        /* DSV4_F32, DSV4_BF16, DSV4_F16, DSV4_FP8R or DSV4_MXFP4 */
  int32_t tail;              /* DSV4_FP8R: bf16 channels at the end; else 0 */
  int64_t pool_cap;          /* pool rows reserved per sequence */
  int32_t *count;            /* [B] pooled entries (state; = len/m after every call) */
} dsv4_stream;

/* A layer's cache: per-sequence token count, the window ring and one or two
 * compressed streams.  All pointers are device memory owned by the caller,
 * zero-initialised (len, counts) before the first append. */
typedef struct {
  int32_t n_seq;             /* B >= 1 */
  int32_t m;                 /* compression stride (CSA 4, HCA 128) */
  int32_t overlap;           /* 1: windows of 2m with stride m (CSA); 0: windows of m (HCA) */
  double rope_theta;         /* one theta for every rotation of the layer */
  const int64_t *pos0;       /* [B] or NULL */
  int32_t *len;              /* [B] tokens appended so far (state) */
  /* window ring of K=V rows, rotated at their positions; win_cap = 0: none */
  void *win;                 /* [B, win_cap] rows of win_dtype (DSV4_F32/BF16/F16/FP8R) */
  float *win_scale;          /* DSV4_FP8R: [B, win_cap] */
  int32_t win_dtype, win_tail, win_cap;
  int32_t win_dim;           /* K=V channels (the kv stream's dim) */
  int32_t win_rope_dim;      /* trailing channels rotated at the token's position */
  int32_t *win_count;        /* [B] state: min(len, win_cap) */
  int32_t *win_first;        /* [B] state: len - win_count */
  dsv4_stream kv;            /* the K=V compressed stream */
  dsv4_stream idx;           /* indexer keys (CSA); idx.dim = 0: absent (HCA) */
} dsv4_cache;

/* dsv4_cache_append -- append up to n tokens to every sequence of a cache.
 * Sequence b takes n_new[b] (<= n; n_new NULL: n) tokens, L_b = len[b] first:
 * token L_b + i comes from row i of the inputs.  The newest win_cap of them
 * are rotated at pos0[b] + token and quantised into the window ring; every
 * entry whose window closes (s with (s+1)m <= L_b + n_new[b]) is pooled from
 * the buffer and the inputs as dsv4_compress does, rotated at pos0[b] + s*m
 * (kv stream) and quantised as dsv4_quantize does; the newest span tokens go
 * to the buffers; len, count, win_count and win_first advance.  Prefill into an
 * empty cache and one decode step are the same call (n = S, or n = 1).
 *   kv            : [B, n, win_dim]       (may be NULL when win_cap = 0)
 *   kv_c, kv_z    : [B, n, kv.dim]
 *   idx_c, idx_z  : [B, n, idx.dim]        (NULL when idx.dim = 0)
 *   in_dtype      : DSV4_F32 or DSV4_BF16 for every input
 *   n_new         : [B] int32 device, or NULL
 * The caller keeps pool_cap >= (len + n_new)/m; entries past pool_cap are not
 * written (count stops at pool_cap).  With DSV4_FP8R the window and pool rows
 * are 576-byte rows for dim 512 / tail 64.  The window ring is read back by
 * the attention calls as a dsv4_rows window with ring = 1, seq_stride =
 * win_cap, count = win_count, first_tok = win_first. */
int dsv4_cache_append(const dsv4_cache *cache, int32_t n, const int32_t *n_new, const void *kv,
                      const void *kv_c, const void *kv_z, const void *idx_c, const void *idx_z,
                      int32_t in_dtype, hipStream_t stream);

/* dsv4_linear -- the projections around the attention core: Y = X W^T.
 * HF DeepSeek-V4 page, "Hybrid attention": kv_proj makes the single K=V head,
 * and the output goes through the grouped low-rank projection (o_groups head
 * groups, each to o_lora_rank by its own weight, then o_b_proj to
 * hidden_size); llm-atlas config: hidden_size 4096, q_lora_rank 1024,
 * o_groups 8, o_lora_rank 1024.  For g < groups, m < M, n < N:
 *   y[g*y_group_stride + m*ldy + n] =
 *       sum_{k<K} x[g*x_group_stride + m*ldx + k] * w[g*w_group_stride + n*ldw + k]
 * accumulated in fp32.  x and w are bfloat16 (row-major, K contiguous: weights
 * stored [out, in]); y is y_dtype (DSV4_F32, DSV4_BF16 or DSV4_F16).  Strides
 * are in elements.  K must be a multiple of 64; x, w 16-byte aligned with row
 * and group strides that are multiples of 8.  groups = 1 with zero group
 * strides is one plain product; the grouped output projection is groups = 8
 * with x the attention output viewed as [T, 8, 4096] (x_group_stride 4096,
 * ldx 32768). */
int dsv4_linear(const void *x, int64_t ldx, const void *w, int64_t ldw, void *y, int64_t ldy, int32_t y_dtype,
                int32_t M, int32_t N, int32_t K, int32_t groups, int64_t x_group_stride,
                int64_t w_group_stride, int64_t y_group_stride, hipStream_t stream);

/* Thread-local description of the last error (empty string after success). */
const char *dsv4_last_error(void);

/* Library version string. */
const char *dsv4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DSV4_H */
