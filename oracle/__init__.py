"""Plain fp64 CPU oracle for the DeepSeek-V4 CSA/HCA attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` import this package.  It shares no code with the
HIP library: it has its own C source (``dsv4_oracle.c``), its own storage
decoders and its own dtype codes.

Two independent formulations live here:

* formulation A -- ``dsv4_oracle.c``: scalar fp64 loops, one query row at a time
  (wrapped by the functions in this module);
* formulation B -- ``mask_oracle.py``: numpy fp64 on the HF eager layout, i.e. a
  ``cat([sliding_causal_mask, block_bias], -1)`` additive mask over gathered keys
  (HF DeepSeek-V4 page, "Attention mask layout").

Every function names the passage of the pages it follows; the readings taken
where the pages are silent are listed in the C source beside each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dsv4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

OR_F32, OR_BF16, OR_FP8R, OR_MXFP4, OR_F64, OR_F16 = 0, 1, 2, 3, 4, 5
_KIND = {"f32": OR_F32, "bf16": OR_BF16, "fp8r": OR_FP8R, "mxfp4": OR_MXFP4, "f64": OR_F64, "f16": OR_F16}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def build_sanitized(outdir: str) -> str:
    """The oracle built with clang's AddressSanitizer and UndefinedBehaviorSanitizer
    (the runtime shared with the library's sanitizer build, so one process can
    load both).  Load it by setting DSV4_ORACLE_LIB."""
    clang = "/opt/rocm/lib/llvm/bin/clang"
    os.makedirs(outdir, exist_ok=True)
    out = os.path.join(outdir, "liboracle_san.so")
    libdir = "/opt/rocm/lib/llvm/lib"
    subprocess.check_call([clang, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-shared-libsan", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall", "-o", out, _SRC,
                           "-lm", f"-L{libdir}", f"-Wl,-rpath,{libdir}"])
    return out


class _Rows(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("row_scale", ctypes.c_void_p),
                ("blk_scale", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("tail", ctypes.c_int32),
                ("seq_stride", ctypes.c_int64), ("count", ctypes.c_void_p),
                ("first_tok", ctypes.c_void_p)]


_lib = None


def _L():
    global _lib
    if _lib is None:
        # DSV4_ORACLE_LIB names another build (the sanitizer build of build_sanitized)
        _lib = ctypes.CDLL(os.environ.get("DSV4_ORACLE_LIB") or build())
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        _lib.or_decode.argtypes = [P, I, I64, I, I, P, P, P]
        _lib.or_rope.argtypes = [P, I64, I, I, P, D, I]
        _lib.or_compress.argtypes = [P, P, I, P, I, I, I, I, I, I, D, P, P]
        _lib.or_index_scores.argtypes = [I, P, P, P, P, I, P, I, I, P, I, D, P, I]
        _lib.or_topk.argtypes = [I, P, I, P, I, P]
        _lib.or_attn.argtypes = [I, P, P, P, P, I, I, I, P, I, P, I, P, I, I, P, D, I, D, P]
        _lib.or_e4m3_to_f64.argtypes = [ctypes.c_uint8]
        _lib.or_e4m3_to_f64.restype = D
        _lib.or_e2m1_to_f64.argtypes = [ctypes.c_uint8]
        _lib.or_e2m1_to_f64.restype = D
        _lib.or_f16_to_f64.argtypes = [ctypes.c_uint16]
        _lib.or_f16_to_f64.restype = D
        _lib.or_e8m0_to_f64.argtypes = [ctypes.c_uint8]
        _lib.or_e8m0_to_f64.restype = D
        _lib.or_quantize_fp8r.argtypes = [I64, I, I, P, P, P]
        _lib.or_quantize_mxfp4.argtypes = [I64, I, P, P, P]
        _lib.or_num_threads.restype = I
        _lib.or_set_num_threads.argtypes = [I]
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def num_threads() -> int:
    return _L().or_num_threads()


def set_num_threads(n: int) -> None:
    _L().or_set_num_threads(int(n))


# ---------------------------------------------------------------- decoders
def e4m3_to_f64(code: int) -> float:
    """OCP FP8 E4M3 (fn) decode of one byte."""
    return _L().or_e4m3_to_f64(code)


def e2m1_to_f64(code: int) -> float:
    """OCP MX E2M1 decode of one nibble."""
    return _L().or_e2m1_to_f64(code)


def f16_to_f64(code: int) -> float:
    """IEEE binary16 decode of one 16-bit pattern."""
    return _L().or_f16_to_f64(code)


def e8m0_to_f64(code: int) -> float:
    """OCP MX E8M0 shared-scale decode."""
    return _L().or_e8m0_to_f64(code)


def decode(rows) -> np.ndarray:
    """Decode a stored row set (see ``dsv4_synth.RowSet``) to fp64 [B, rows, dim]."""
    B, n = rows.n_seq, rows.rows_per_seq
    out = np.empty((B * n, rows.dim), dtype=np.float64)
    data = np.ascontiguousarray(rows.data)
    rs = _c(rows.row_scale, np.float32)
    bs = _c(rows.blk_scale, np.uint8)
    _L().or_decode(data.ctypes.data, _KIND[rows.kind], B * n, rows.dim, rows.tail,
                   _p(rs), _p(bs), out.ctypes.data)
    return out.reshape(B, n, rows.dim)


# ---------------------------------------------------------------- encoders
def quantize_fp8r(x: np.ndarray, tail: int):
    """Q1 -- FP8 KV row storage (insight.ai.kr deep dive: FP8 cache, RoPE
    channels in BF16).  x [..., dim] float32 (values taken as fp32).
    Returns (rows [..., (dim-tail) + 2*tail] uint8, scales [...] float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    dim = x.shape[-1]
    n = x.size // dim
    rows = np.empty((n, (dim - tail) + 2 * tail), np.uint8)
    sc = np.empty(n, np.float32)
    _L().or_quantize_fp8r(n, dim, tail, x.ctypes.data, rows.ctypes.data, sc.ctypes.data)
    return rows.reshape(*x.shape[:-1], -1), sc.reshape(x.shape[:-1])


def quantize_mxfp4(x: np.ndarray):
    """Q2 -- MXFP4 (MarkTechPost: FP4 on the indexer query/key path).
    x [..., dim] float32, dim % 32 == 0.  Returns (nibbles [..., dim/2] uint8,
    E8M0 scales [..., dim/32] uint8)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    dim = x.shape[-1]
    n = x.size // dim
    rows = np.empty((n, dim // 2), np.uint8)
    sc = np.empty((n, dim // 32), np.uint8)
    _L().or_quantize_mxfp4(n, dim, x.ctypes.data, rows.ctypes.data, sc.ctypes.data)
    return rows.reshape(*x.shape[:-1], -1), sc.reshape(*x.shape[:-1], -1)


# ---------------------------------------------------------------- wrapped steps
def rope(x: np.ndarray, pos: np.ndarray, rope_dim: int, theta: float, sign: int) -> np.ndarray:
    """O1 -- partial interleaved RoPE of the last rope_dim channels.

    HF DeepSeek-V4 page, "Hybrid attention": partial RoPE on the trailing
    qk_rope_head_dim channels; the output slice is rotated back at -p.
    x: [..., dim] (any float); pos: one position per row.  Returns fp64."""
    x = np.array(x, dtype=np.float64, copy=True)
    dim = x.shape[-1]
    flat = x.reshape(-1, dim)
    pos = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, dtype=np.float64).reshape(-1, 1),
                                               (flat.shape[0], 1)).reshape(-1))
    _L().or_rope(flat.ctypes.data, flat.shape[0], dim, rope_dim, pos.ctypes.data, float(theta), int(sign))
    return flat.reshape(x.shape)


def compress(c: np.ndarray, z: np.ndarray, bias: np.ndarray, m: int, overlap: bool,
             rope_dim: int = 0, theta: float = 10000.0, pos0: Optional[np.ndarray] = None,
             kind: str = "f32") -> np.ndarray:
    """O2 -- softmax-gated pooling with a learned position bias.

    HF page "Hybrid attention" (CSA overlapping windows, HCA non-overlapping);
    insight.ai.kr CSA paragraph (softmax-gated pooling, learned position bias).
    c, z: [B, S, dim] stored as ``kind`` ('f32' float32 values, 'bf16' uint16
    bit patterns, 'f64'); bias [window, dim].  Returns fp64 [B, S//m, dim]."""
    dt = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[kind]
    c = _c(c, dt)
    z = _c(z, dt)
    B, S, dim = c.shape
    width = 2 * m if overlap else m
    bias = _c(bias, np.float64)
    assert bias.shape == (width, dim), bias.shape
    N = S // m
    out = np.zeros((B, N, dim), dtype=np.float64)
    p0 = _c(pos0 if pos0 is not None else np.zeros(B), np.int64)
    _L().or_compress(c.ctypes.data, z.ctypes.data, _KIND[kind], bias.ctypes.data, B, S, dim, m,
                     1 if overlap else 0, rope_dim, float(theta), p0.ctypes.data, out.ctypes.data)
    return out


@dataclass
class _RowsHold:
    st: _Rows
    keep: tuple


def _rows(rs) -> _RowsHold:
    """Marshal a ``dsv4_synth.RowSet`` (numpy arrays) into the oracle struct."""
    data = np.ascontiguousarray(rs.data)
    rsc = _c(rs.row_scale, np.float32)
    bsc = _c(rs.blk_scale, np.uint8)
    cnt = _c(rs.count, np.int32)
    ft = _c(rs.first_tok, np.int32)
    st = _Rows(data.ctypes.data, _p(rsc), _p(bsc), _KIND[rs.kind], rs.dim, rs.tail,
               rs.rows_per_seq, cnt.ctypes.data, _p(ft))
    return _RowsHold(st, (data, rsc, bsc, cnt, ft))


def n_visible(tok, m: int, count) -> np.ndarray:
    """O3 -- entries visible to token t: min(count, (t+1)//m) (HF page, mask layout)."""
    return np.minimum((np.asarray(tok, dtype=np.int64) + 1) // m, np.asarray(count, dtype=np.int64))


def index_scores(q_seq, q_tok, q_idx, q_kind: str, w, kpool, m: int, score_scale: float,
                 nmax: Optional[int] = None, q_scale=None) -> np.ndarray:
    """O4 -- Lightning Indexer scores scale * sum_h w[t,h] * ReLU(q_I[t,h] . k_I[s]).

    insight.ai.kr CSA paragraph (ReLU-scored multi-head dot products);
    MarkTechPost summary (MXFP4 on the indexer query/key path).
    q_idx: [n_q, H, Di] stored as q_kind (mxfp4: packed bytes [n_q, H, Di/2]
    with q_scale [n_q, H, Di/32]).  Returns fp64 [n_q, nmax], -inf where s >= n(t)."""
    q_seq = _c(q_seq, np.int32)
    q_tok = _c(q_tok, np.int32)
    n_q = q_seq.shape[0]
    H = w.shape[-1]
    Di = kpool.dim
    w = _c(w, np.float64).reshape(n_q, H)
    dt = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64, "mxfp4": np.uint8}[q_kind]
    qd = _c(q_idx, dt)
    qs = _c(q_scale, np.uint8)
    if nmax is None:
        nmax = int(np.max(kpool.count)) if n_q else 0
    out = np.empty((n_q, max(nmax, 1)), dtype=np.float64)
    hold = _rows(kpool)
    _L().or_index_scores(n_q, q_seq.ctypes.data, q_tok.ctypes.data, qd.ctypes.data, _p(qs),
                         _KIND[q_kind], w.ctypes.data, H, Di, ctypes.byref(hold.st), m,
                         float(score_scale), out.ctypes.data, nmax)
    return out[:, :nmax]


def topk(scores: np.ndarray, n_valid, k: int) -> np.ndarray:
    """O5 -- top-k with ties to the lower index, ascending output, -1 fill.

    HF page "Attention mask layout", CSA paragraph (top index_topk blocks,
    -1 sentinel before the first window closes)."""
    scores = _c(scores, np.float64)
    n_q, nmax = scores.shape
    nv = _c(n_valid, np.int32)
    out = np.empty((n_q, max(k, 1)), dtype=np.int32)
    _L().or_topk(n_q, scores.ctypes.data, nmax, nv.ctypes.data, k, out.ctypes.data)
    return out[:, :k]


def attn(q_seq, q_tok, pos0, q, q_kind: str, win, W: int, pool, mode: str, idx=None,
         k: int = 0, m: int = 1, sinks=None, sm_scale: float = 1.0, rope_dim: int = 0,
         theta: float = 10000.0) -> np.ndarray:
    """O6 (mode 'csa') / O7 (mode 'hca') -- shared K=V MQA with sink and window.

    HF page "Hybrid attention" backbone bullets (shared K=V, partial RoPE with
    the inverse rotation of the output, per-head sink, sliding-window branch
    concatenated with the compressed entries) and "Attention mask layout".
    q: [n_q, H, D] stored as q_kind ('f32' | 'bf16' | 'f64').  win/pool are
    ``dsv4_synth.RowSet`` or None.  Returns fp64 [n_q, H, D]."""
    q_seq = _c(q_seq, np.int32)
    q_tok = _c(q_tok, np.int32)
    n_q = q_seq.shape[0]
    dt = {"f32": np.float32, "bf16": np.uint16, "f64": np.float64}[q_kind]
    qd = _c(q, dt)
    H, D = qd.shape[-2], qd.shape[-1]
    p0 = _c(pos0, np.int64)
    hw = _rows(win) if win is not None else None
    hp = _rows(pool) if pool is not None else None
    if mode == "csa":
        idx = _c(idx, np.int32)
        k = idx.shape[1] if idx is not None else 0
    sk = _c(sinks, np.float64)
    out = np.zeros((n_q, H, D), dtype=np.float64)
    _L().or_attn(n_q, q_seq.ctypes.data, q_tok.ctypes.data, _p(p0), qd.ctypes.data, _KIND[q_kind],
                 H, D, ctypes.byref(hw.st) if hw else None, W,
                 ctypes.byref(hp.st) if hp else None, 0 if mode == "csa" else 1,
                 _p(idx) if mode == "csa" else None, k, m, _p(sk), float(sm_scale),
                 rope_dim, float(theta), out.ctypes.data)
    return out


# ---------------------------------------------------------------- projections
def linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """P1 -- one projection y = x W^T, fp64 (weights stored [out, in]).

    HF DeepSeek-V4 page, "Hybrid attention": kv_proj makes the single K=V head
    (and the other projections around the core are plain linear maps of the
    hidden states).  x: [..., K] (any float, taken exactly), w: [N, K].
    Returns fp64 [..., N]."""
    return np.asarray(x, np.float64) @ np.asarray(w, np.float64).T


def grouped_linear(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """P2 -- grouped projection, fp64.

    HF DeepSeek-V4 page, "Hybrid attention", grouped low-rank output
    projection: the heads are split into o_groups groups and each group's
    concatenated head outputs go through its own [o_lora_rank, group width]
    weight.  x: [M, G*K] (group g = columns gK .. gK+K-1), w: [G, N, K].
    Returns fp64 [M, G*N] (group g's outputs at columns gN .. gN+N-1)."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    G, N, K = w.shape
    assert x.shape[-1] == G * K
    return np.concatenate([x[:, g * K:(g + 1) * K] @ w[g].T for g in range(G)], axis=-1)
