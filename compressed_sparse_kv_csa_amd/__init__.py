"""Python binding of libdsv4 (the gfx950 CSA/HCA attention hot path).

Argument marshalling only: every function takes torch tensors that live in
device memory, checks shapes and dtypes, and calls the C entry point of the
same name in ``libdsv4.so`` on ``torch.cuda.current_stream()``.  No step of the
path is computed here, and nothing falls back to the CPU: if the library is
missing the import of a function raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# DSV4_LIB names another build of the library (the host sanitizer build of
# build.build_sanitized is loaded this way); the in-tree libdsv4.so otherwise
LIB_PATH = os.environ.get("DSV4_LIB") or os.path.join(HERE, "libdsv4.so")

DSV4_F32, DSV4_BF16, DSV4_FP8R, DSV4_MXFP4, DSV4_F16 = 0, 1, 2, 3, 4
DSV4_OK, DSV4_EINVAL, DSV4_ENOTSUP, DSV4_EHIP, DSV4_EWORKSPACE = 0, -1, -2, -3, -4

EXPORTS = ["dsv4_compress", "dsv4_rope", "dsv4_index_topk_workspace", "dsv4_index_topk",
           "dsv4_attn_workspace", "dsv4_sparse_attn", "dsv4_hca_attn", "dsv4_set_batch_invariant", "dsv4_set_diagnostics", "dsv4_read_diagnostics",
           "dsv4_quantize", "dsv4_cache_append", "dsv4_linear", "dsv4_last_error", "dsv4_version",
           "dsv4_index_topk_noalloc"]
NOALLOC_SCRATCH_BYTES = 16 << 20   # DSV4_NOALLOC_SCRATCH_BYTES in include/dsv4.h


class Dsv4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dsv4 error {code}: {msg}")
        self.code = code


class Queries(ctypes.Structure):
    _fields_ = [("n_rows", ctypes.c_int32), ("n_seq", ctypes.c_int32), ("seq", ctypes.c_void_p),
                ("tok", ctypes.c_void_p), ("pos0", ctypes.c_void_p)]


class Rows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("row_scale", ctypes.c_void_p), ("blk_scale", ctypes.c_void_p),
                ("dtype", ctypes.c_int32), ("dim", ctypes.c_int32), ("tail", ctypes.c_int32),
                ("seq_stride", ctypes.c_int64), ("count", ctypes.c_void_p), ("first_tok", ctypes.c_void_p),
                ("ring", ctypes.c_int32)]


class Stream(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("pos_bias", ctypes.c_void_p),
                ("buf", ctypes.c_void_p), ("pool", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
                ("blk_scale", ctypes.c_void_p), ("pool_dtype", ctypes.c_int32), ("tail", ctypes.c_int32),
                ("pool_cap", ctypes.c_int64), ("count", ctypes.c_void_p)]


class Cache(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("m", ctypes.c_int32), ("overlap", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("pos0", ctypes.c_void_p), ("len", ctypes.c_void_p),
                ("win", ctypes.c_void_p), ("win_scale", ctypes.c_void_p), ("win_dtype", ctypes.c_int32),
                ("win_tail", ctypes.c_int32), ("win_cap", ctypes.c_int32), ("win_dim", ctypes.c_int32),
                ("win_rope_dim", ctypes.c_int32), ("win_count", ctypes.c_void_p), ("win_first", ctypes.c_void_p),
                ("kv", Stream), ("idx", Stream)]


_lib = None


def lib():
    """Load libdsv4.so (torch is imported first so that one HIP runtime serves both)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m compressed_sparse_kv_csa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, F, D, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                 ctypes.c_double, ctypes.c_size_t)
        L.dsv4_compress.argtypes = [P, P, I32, P, I32, I32, I32, I32, I32, I32, D, P, P, I32, P]
        L.dsv4_rope.argtypes = [P, I32, P, I32, I64, I32, I32, P, D, I32, P]
        L.dsv4_index_topk_workspace.argtypes = [I32, I64, I32]
        L.dsv4_index_topk_workspace.restype = SZ
        L.dsv4_index_topk.argtypes = [P, P, P, I32, P, I32, I32, P, I32, I32, F, P, P, P, SZ, P]
        L.dsv4_index_topk_noalloc.argtypes = [P, P, P, I32, P, I32, I32, P, I32, I32, F, P, P, P]
        L.dsv4_attn_workspace.argtypes = [I32, I32, I32, I64]
        L.dsv4_attn_workspace.restype = SZ
        L.dsv4_sparse_attn.argtypes = [P, P, I32, I32, I32, P, I32, P, P, I32, P, F, I32, D, P, I32, P, SZ, P]
        L.dsv4_hca_attn.argtypes = [P, P, I32, I32, I32, P, I32, P, I32, P, F, I32, D, P, I32, P, SZ, P]
        L.dsv4_set_batch_invariant.argtypes = [I32]
        L.dsv4_set_diagnostics.argtypes = [I32]
        L.dsv4_read_diagnostics.argtypes = [P, I32]
        L.dsv4_quantize.argtypes = [P, I32, I64, I32, I32, P, P, P, I32, P]
        L.dsv4_cache_append.argtypes = [P, I32, P, P, P, P, P, P, I32, P]
        L.dsv4_linear.argtypes = [P, I64, P, I64, P, I64, I32, I32, I32, I32, I32, I64, I64, I64, P]
        L.dsv4_last_error.restype = ctypes.c_char_p
        L.dsv4_version.restype = ctypes.c_char_p
        for name in EXPORTS:
            getattr(L, name).restype = getattr(L, name).restype or ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != DSV4_OK:
        raise Dsv4Error(rc, lib().dsv4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("dsv4 tensors must live in device memory")
    if not t.is_contiguous():
        raise ValueError("dsv4 tensors must be contiguous")
    return t.data_ptr()


def _ptr_rows(t: torch.Tensor):
    """Pointer of a 2-D tensor whose rows may be strided (unit column stride)."""
    if not t.is_cuda:
        raise ValueError("dsv4 tensors must live in device memory")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a 2-D tensor with contiguous rows")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


_CODES = {torch.float32: DSV4_F32, torch.bfloat16: DSV4_BF16, torch.float16: DSV4_F16}


def _code(t: torch.Tensor) -> int:
    if t.dtype not in _CODES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _CODES[t.dtype]


# ------------------------------------------------------------------ descriptors
@dataclass
class QueryRows:
    """Device arrays describing query rows (sequence, token) and per-sequence pos0."""
    seq: torch.Tensor      # [T] int32
    tok: torch.Tensor      # [T] int32
    pos0: Optional[torch.Tensor]   # [B] int64
    n_seq: int

    def c(self) -> Queries:
        return Queries(self.seq.numel(), self.n_seq, _ptr(self.seq), _ptr(self.tok), _ptr(self.pos0))

    @staticmethod
    def prefill(n_seq: int, seq_len: int, pos0: Optional[torch.Tensor] = None, device="cuda") -> "QueryRows":
        seq = torch.arange(n_seq, dtype=torch.int32, device=device).repeat_interleave(seq_len)
        tok = torch.arange(seq_len, dtype=torch.int32, device=device).repeat(n_seq)
        return QueryRows(seq, tok, pos0, n_seq)

    @staticmethod
    def decode(lengths: torch.Tensor, pos0: Optional[torch.Tensor] = None) -> "QueryRows":
        B = lengths.numel()
        seq = torch.arange(B, dtype=torch.int32, device=lengths.device)
        return QueryRows(seq, (lengths - 1).to(torch.int32), pos0, B)


@dataclass
class RowStore:
    """Per-sequence rows in device memory (see dsv4_rows in include/dsv4.h).

    data: [B, stride, row_bytes] uint8, or a typed tensor [B, stride, dim]."""
    data: torch.Tensor
    dtype: int
    dim: int
    count: torch.Tensor                      # [B] int32
    tail: int = 0
    row_scale: Optional[torch.Tensor] = None  # [B, stride] f32
    blk_scale: Optional[torch.Tensor] = None  # [B, stride, dim/32] u8
    first_tok: Optional[torch.Tensor] = None  # [B] int32
    ring: bool = False                        # window ring: token j at row j mod stride

    @property
    def stride(self) -> int:
        return self.data.shape[1]

    def c(self) -> Rows:
        return Rows(_ptr(self.data), _ptr(self.row_scale), _ptr(self.blk_scale), self.dtype, self.dim,
                    self.tail, self.stride, _ptr(self.count), _ptr(self.first_tok), 1 if self.ring else 0)


def row_bytes(dtype: int, dim: int, tail: int = 0) -> int:
    """Bytes of one stored row (see the storage types in include/dsv4.h)."""
    return {DSV4_F32: 4 * dim, DSV4_BF16: 2 * dim, DSV4_F16: 2 * dim,
            DSV4_FP8R: (dim - tail) + 2 * tail, DSV4_MXFP4: dim // 2}[dtype]


class DecodeCache:
    """Device state of one compressed-attention layer's cache (dsv4_cache in
    include/dsv4.h): token counts, the window ring of K=V rows and one
    (HCA) or two (CSA: K=V and indexer keys) compressed streams, each with
    its buffer of the newest tokens, pool and count.  Tensors are allocated
    here (torch, device memory); every update runs in dsv4_cache_append."""

    def __init__(self, n_seq: int, m: int, overlap: bool, kv_dim: int, kv_bias: torch.Tensor, pool_cap: int,
                 win_cap: int, rope_dim: int = 0, rope_theta: float = 10000.0, kv_dtype: int = DSV4_FP8R,
                 kv_tail: int = 0, win_dtype: Optional[int] = None, idx_dim: int = 0,
                 idx_bias: Optional[torch.Tensor] = None, idx_dtype: int = DSV4_MXFP4,
                 pos0: Optional[torch.Tensor] = None, device="cuda"):
        span = 2 * m if overlap else m
        self.n_seq, self.m, self.overlap, self.span = n_seq, m, bool(overlap), span
        self.rope_theta, self.pos0 = float(rope_theta), pos0
        i32 = dict(dtype=torch.int32, device=device)
        self.len = torch.zeros(n_seq, **i32)
        self.win_dtype = kv_dtype if win_dtype is None else win_dtype
        self.win_tail = kv_tail if self.win_dtype == DSV4_FP8R else 0
        self.win_cap, self.kv_dim, self.rope_dim = win_cap, kv_dim, rope_dim
        self.win = torch.zeros(n_seq, max(win_cap, 1), row_bytes(self.win_dtype, kv_dim, self.win_tail),
                               dtype=torch.uint8, device=device)
        self.win_scale = (torch.zeros(n_seq, max(win_cap, 1), dtype=torch.float32, device=device)
                          if self.win_dtype == DSV4_FP8R else None)
        self.win_count = torch.zeros(n_seq, **i32)
        self.win_first = torch.zeros(n_seq, **i32)
        self.kv = self._stream(kv_dim, rope_dim, kv_bias, kv_dtype, kv_tail, pool_cap, device)
        self.idx = (self._stream(idx_dim, 0, idx_bias, idx_dtype, 0, pool_cap, device)
                    if idx_dim else None)

    def _stream(self, dim, rope_dim, bias, dtype, tail, cap, device):
        assert bias is not None and tuple(bias.shape) == (self.span, dim) and bias.dtype == torch.float32
        st = dict(dim=dim, rope_dim=rope_dim, bias=bias.contiguous(), dtype=dtype, tail=tail,
                  buf=torch.zeros(self.n_seq, self.span, 2, dim, dtype=torch.float32, device=device),
                  pool=torch.zeros(self.n_seq, max(cap, 1), row_bytes(dtype, dim, tail), dtype=torch.uint8,
                                   device=device),
                  row_scale=(torch.zeros(self.n_seq, max(cap, 1), dtype=torch.float32, device=device)
                             if dtype == DSV4_FP8R else None),
                  blk_scale=(torch.zeros(self.n_seq, max(cap, 1), dim // 32, dtype=torch.uint8, device=device)
                             if dtype == DSV4_MXFP4 else None),
                  cap=cap, count=torch.zeros(self.n_seq, dtype=torch.int32, device=device))
        return st

    @staticmethod
    def _c_stream(st) -> Stream:
        if st is None:
            return Stream()
        return Stream(st["dim"], st["rope_dim"], _ptr(st["bias"]), _ptr(st["buf"]), _ptr(st["pool"]),
                      _ptr(st["row_scale"]), _ptr(st["blk_scale"]), st["dtype"], st["tail"], st["cap"],
                      _ptr(st["count"]))

    def c(self) -> Cache:
        return Cache(self.n_seq, self.m, 1 if self.overlap else 0, self.rope_theta, _ptr(self.pos0),
                     _ptr(self.len), _ptr(self.win), _ptr(self.win_scale), self.win_dtype, self.win_tail,
                     self.win_cap, self.kv_dim, self.rope_dim, _ptr(self.win_count), _ptr(self.win_first),
                     self._c_stream(self.kv), self._c_stream(self.idx))

    def append(self, kv: Optional[torch.Tensor], kv_c: torch.Tensor, kv_z: torch.Tensor,
               idx_c: Optional[torch.Tensor] = None, idx_z: Optional[torch.Tensor] = None,
               n_new: Optional[torch.Tensor] = None, stream=None) -> None:
        """dsv4_cache_append: inputs [B, n, dim], all float32 or all bfloat16;
        n_new [B] int32 (tokens taken per sequence, <= n) or None."""
        B, n, _ = kv_c.shape
        assert B == self.n_seq
        ins = [t for t in (kv, kv_c, kv_z, idx_c, idx_z) if t is not None]
        code = _code(kv_c)
        for t in ins:
            assert t.dtype == kv_c.dtype and t.shape[:2] == (B, n), "inputs: one dtype, shape [B, n, dim]"
        cs = self.c()
        _check(lib().dsv4_cache_append(ctypes.byref(cs), n, _ptr(n_new), _ptr(kv), _ptr(kv_c), _ptr(kv_z),
                                       _ptr(idx_c), _ptr(idx_z), code, _stream(stream)))

    def window(self) -> RowStore:
        """The window ring as attention calls read it."""
        return RowStore(self.win, self.win_dtype, self.kv_dim, self.win_count, tail=self.win_tail,
                        row_scale=self.win_scale, first_tok=self.win_first, ring=True)

    @staticmethod
    def _pool(st) -> RowStore:
        return RowStore(st["pool"], st["dtype"], st["dim"], st["count"], tail=st["tail"],
                        row_scale=st["row_scale"], blk_scale=st["blk_scale"])

    def kv_pool(self) -> RowStore:
        return self._pool(self.kv)

    def idx_pool(self) -> RowStore:
        assert self.idx is not None, "this cache has no indexer stream"
        return self._pool(self.idx)


# ------------------------------------------------------------------ entry points
def dsv4_compress(c: torch.Tensor, z: torch.Tensor, pos_bias: torch.Tensor, m: int, overlap: bool,
                  rope_dim: int = 0, rope_theta: float = 10000.0, pos0: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """KV compressor: c, z [B, S, dim] -> pool [B, S//m, dim]."""
    B, S, dim = c.shape
    assert z.shape == c.shape and z.dtype == c.dtype
    assert pos_bias.dtype == torch.float32 and pos_bias.shape == ((2 * m if overlap else m), dim)
    odt = out_dtype or c.dtype
    if out is None:
        out = torch.empty(B, S // m, dim, dtype=odt, device=c.device)
    _check(lib().dsv4_compress(_ptr(c), _ptr(z), _code(c), _ptr(pos_bias), B, S, dim, m, int(bool(overlap)),
                               rope_dim, float(rope_theta), _ptr(pos0), _ptr(out), _code(out), _stream()))
    return out


def dsv4_rope(x: torch.Tensor, pos: torch.Tensor, rope_dim: int, rope_theta: float, inverse: bool = False,
              out: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None) -> torch.Tensor:
    """Partial interleaved RoPE of the last rope_dim channels; x [..., dim], pos [rows] int64."""
    dim = x.shape[-1]
    n = x.numel() // dim
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    assert pos.dtype == torch.int64 and pos.numel() == n and out.numel() == x.numel()
    _check(lib().dsv4_rope(_ptr(x), _code(x), _ptr(out), _code(out), n, dim, rope_dim, _ptr(pos),
                           float(rope_theta), int(bool(inverse)), _stream()))
    return out


def dsv4_index_topk(q: QueryRows, q_idx: torch.Tensor, w: torch.Tensor, k_pool: RowStore, m: int, topk: int,
                    score_scale: float, q_idx_scale: Optional[torch.Tensor] = None, q_dtype: Optional[int] = None,
                    want_scores: bool = False, ws: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None):
    """Lightning Indexer + top-k.  Returns idx [T, topk] int32 (and scores)."""
    T = q.seq.numel()
    H = w.shape[-1]
    if q_dtype is None:
        q_dtype = DSV4_MXFP4 if q_idx.dtype == torch.uint8 else _code(q_idx)
    Di = k_pool.dim
    idx = out if out is not None else torch.empty(T, topk, dtype=torch.int32, device=w.device)
    assert idx.dtype == torch.int32 and idx.shape == (T, topk)
    sc = torch.empty(T, topk, dtype=torch.float32, device=w.device) if want_scores else None
    need = lib().dsv4_index_topk_workspace(T, k_pool.stride, topk)
    if ws is None or ws.numel() < need:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=w.device)
    qc, kc = q.c(), k_pool.c()
    _check(lib().dsv4_index_topk(ctypes.byref(qc), _ptr(q_idx), _ptr(q_idx_scale), q_dtype, _ptr(w), H, Di,
                                 ctypes.byref(kc), m, topk, float(score_scale), _ptr(idx), _ptr(sc), _ptr(ws),
                                 ws.numel(), _stream()))
    return (idx, sc) if want_scores else idx


def dsv4_index_topk_noalloc(q: QueryRows, q_idx: torch.Tensor, w: torch.Tensor, k_pool: RowStore, m: int,
                            topk: int, score_scale: float, out: torch.Tensor, q_idx_scale: Optional[torch.Tensor] = None,
                            q_dtype: Optional[int] = None, score_out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dsv4_index_topk with the library's static scratch in place of a workspace
    (for callers that cannot allocate).  The caller passes the output idx
    [T, topk] int32 (and optionally score_out [T, topk] float32)."""
    H = w.shape[-1]
    if q_dtype is None:
        q_dtype = DSV4_MXFP4 if q_idx.dtype == torch.uint8 else _code(q_idx)
    assert out.dtype == torch.int32 and out.shape == (q.seq.numel(), topk)
    qc, kc = q.c(), k_pool.c()
    _check(lib().dsv4_index_topk_noalloc(ctypes.byref(qc), _ptr(q_idx), _ptr(q_idx_scale), q_dtype, _ptr(w), H,
                                         k_pool.dim, ctypes.byref(kc), m, topk, float(score_scale), _ptr(out),
                                         _ptr(score_out), _stream()))
    return out


def index_topk_workspace(n_rows: int, pool_stride: int, topk: int, device="cuda") -> torch.Tensor:
    """A workspace tensor large enough for dsv4_index_topk."""
    return torch.empty(max(1, lib().dsv4_index_topk_workspace(n_rows, pool_stride, topk)), dtype=torch.uint8,
                       device=device)


def attn_workspace(n_rows: int, n_heads: int, dim: int, max_rows: int, device="cuda") -> Optional[torch.Tensor]:
    """A workspace tensor for dsv4_sparse_attn / dsv4_hca_attn (None if none is needed)."""
    need = lib().dsv4_attn_workspace(n_rows, n_heads, dim, max_rows)
    return torch.empty(need, dtype=torch.uint8, device=device) if need else None


def _attn_ws(T, H, D, max_rows, device, ws):
    need = lib().dsv4_attn_workspace(T, H, D, max_rows)
    if need == 0:
        return ws, 0
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel()


def dsv4_sparse_attn(q: QueryRows, qv: torch.Tensor, window: Optional[RowStore], W: int, pool: Optional[RowStore],
                     idx: Optional[torch.Tensor], sinks: Optional[torch.Tensor], sm_scale: float, rope_dim: int,
                     rope_theta: float, out_dtype: Optional[torch.dtype] = None,
                     ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """CSA core attention.  qv [T, H, D]; idx [T, topk] int32 (or None: no pool branch)."""
    T, H, D = qv.shape
    topk = 0 if idx is None else idx.shape[1]
    if out is None:
        out = torch.empty(T, H, D, dtype=out_dtype or qv.dtype, device=qv.device)
    ws, nbytes = _attn_ws(T, H, D, W + topk, qv.device, ws)
    qc = q.c()
    wc = window.c() if window is not None else None
    pc = pool.c() if pool is not None else None
    _check(lib().dsv4_sparse_attn(ctypes.byref(qc), _ptr(qv), _code(qv), H, D,
                                  ctypes.byref(wc) if wc is not None else None, W,
                                  ctypes.byref(pc) if pc is not None else None, _ptr(idx), topk, _ptr(sinks),
                                  float(sm_scale), rope_dim, float(rope_theta), _ptr(out), _code(out),
                                  _ptr(ws), nbytes, _stream()))
    return out


def dsv4_hca_attn(q: QueryRows, qv: torch.Tensor, window: Optional[RowStore], W: int, pool: Optional[RowStore],
                  m: int, sinks: Optional[torch.Tensor], sm_scale: float, rope_dim: int, rope_theta: float,
                  out_dtype: Optional[torch.dtype] = None, ws: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """HCA core attention: dense over visible pool entries plus the window."""
    T, H, D = qv.shape
    if out is None:
        out = torch.empty(T, H, D, dtype=out_dtype or qv.dtype, device=qv.device)
    ws, nbytes = _attn_ws(T, H, D, W + (pool.stride if pool is not None else 0), qv.device, ws)
    qc = q.c()
    wc = window.c() if window is not None else None
    pc = pool.c() if pool is not None else None
    _check(lib().dsv4_hca_attn(ctypes.byref(qc), _ptr(qv), _code(qv), H, D,
                               ctypes.byref(wc) if wc is not None else None, W,
                               ctypes.byref(pc) if pc is not None else None, m, _ptr(sinks), float(sm_scale),
                               rope_dim, float(rope_theta), _ptr(out), _code(out), _ptr(ws), nbytes, _stream()))
    return out


def dsv4_linear(x: torch.Tensor, w: torch.Tensor, out_dtype: Optional[torch.dtype] = None,
                groups: int = 1, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Y = X W^T (bf16 in, fp32 accumulate).  groups = 1: x [M, K], w [N, K] ->
    y [M, N].  groups = G: x [M, G*K] (group g = columns g*K .. g*K+K-1),
    w [G, N, K] -> y [M, G*N]."""
    assert x.dtype == torch.bfloat16 and w.dtype == torch.bfloat16, "bf16 operands"
    M = x.shape[0]
    if groups == 1:
        N, K = w.shape
        assert x.shape[-1] == K
        gx = gw = gy = 0
    else:
        G, N, K = w.shape
        assert G == groups and x.shape[-1] == G * K
        gx, gw, gy = K, N * K, N
    y = out if out is not None else torch.empty(M, groups * N, dtype=out_dtype or torch.bfloat16, device=x.device)
    assert y.shape == (M, groups * N)
    _check(lib().dsv4_linear(_ptr_rows(x), x.stride(0), _ptr(w), K, _ptr_rows(y), y.stride(0), _code(y), M, N, K,
                             groups, gx, gw, gy, _stream(stream)))
    return y


def dsv4_quantize(x: torch.Tensor, out_dtype: int, tail: int = 0):
    """Quantise rows x [..., dim] (float32 / bfloat16 / float16) for storage.
    DSV4_FP8R -> (rows uint8 [..., (dim-tail) + 2*tail], row scales float32 [...]);
    DSV4_MXFP4 -> (nibbles uint8 [..., dim/2], E8M0 block scales uint8 [..., dim/32])."""
    x = x.contiguous()
    dim = x.shape[-1]
    lead = tuple(x.shape[:-1])
    n = x.numel() // dim
    if out_dtype == DSV4_FP8R:
        rows = torch.empty(lead + ((dim - tail) + 2 * tail,), dtype=torch.uint8, device=x.device)
        sc = torch.empty(lead, dtype=torch.float32, device=x.device)
        _check(lib().dsv4_quantize(_ptr(x), _code(x), n, dim, tail, _ptr(rows), _ptr(sc), None, out_dtype,
                                   _stream()))
    else:
        rows = torch.empty(lead + (dim // 2,), dtype=torch.uint8, device=x.device)
        sc = torch.empty(lead + (dim // 32,), dtype=torch.uint8, device=x.device)
        _check(lib().dsv4_quantize(_ptr(x), _code(x), n, dim, tail, _ptr(rows), None, _ptr(sc), out_dtype,
                                   _stream()))
    return rows, sc


def dsv4_set_batch_invariant(on: bool) -> bool:
    """Fixed per-query reduction order whatever the batch (see include/dsv4.h).
    Returns the previous setting."""
    return bool(lib().dsv4_set_batch_invariant(int(bool(on))))


DSV4_DIAG_REF_RAISES, DSV4_DIAG_BAD_PICKS, DSV4_DIAG_COUNT = 0, 1, 4


def dsv4_set_diagnostics(on: bool) -> bool:
    """Count softmax reference raises and out-of-range picks in the attention calls
    (see include/dsv4.h).  Returns the previous setting."""
    return bool(lib().dsv4_set_diagnostics(int(bool(on))))


def dsv4_read_diagnostics(reset: bool = False) -> dict:
    """The current GPU's counters after its queued work: {"ref_raises", "bad_picks"}."""
    buf = (ctypes.c_uint64 * DSV4_DIAG_COUNT)()
    _check(lib().dsv4_read_diagnostics(ctypes.addressof(buf), int(bool(reset))))
    return {"ref_raises": int(buf[DSV4_DIAG_REF_RAISES]), "bad_picks": int(buf[DSV4_DIAG_BAD_PICKS])}


def dsv4_last_error() -> str:
    return lib().dsv4_last_error().decode()


def dsv4_version() -> str:
    return lib().dsv4_version().decode()
