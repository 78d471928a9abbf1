"""Formulation B of the oracle: numpy fp64 on the HF eager-attention layout.

TEST INFRASTRUCTURE ONLY (imported by tests/ alone).  It is written
independently of ``dsv4_oracle.c`` and shares nothing with the HIP library.

HF DeepSeek-V4 page, "Attention mask layout": every layer extends the
[S, S] sliding-window causal mask with the compressor's ``block_bias`` along the
key axis (``cat([sliding_causal_mask, block_bias], -1)``) and runs eager
attention over the concatenated keys.  CSA gathers each query's picks into a
flat [S*k] key axis where query t owns columns [S + t*k, S + (t+1)*k) and every
other compressor column is -inf (the -1 sentinel masks its slot); HCA appends
the N pooled entries and lets query t see entry w iff w < (t+1)//m.

Everything is whole-matrix numpy (masks, einsum, complex rotation), so a slip in
either formulation shows up as a disagreement between the two.
"""
from __future__ import annotations

import numpy as np


def rope_complex(x: np.ndarray, pos: np.ndarray, rope_dim: int, theta: float, sign: int) -> np.ndarray:
    """Partial interleaved RoPE written with complex numbers: the pair
    (x[2i], x[2i+1]) of the trailing rope_dim channels is the complex number
    x[2i] + 1j*x[2i+1], multiplied by exp(1j*sign*pos*theta**(-2i/R)).
    x: [..., dim]; pos broadcastable to x.shape[:-1]."""
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    dim = x.shape[-1]
    tail = x[..., dim - rope_dim:]
    zc = tail[..., 0::2] + 1j * tail[..., 1::2]
    inv = theta ** (-np.arange(rope_dim // 2, dtype=np.float64) * 2.0 / rope_dim)
    ang = sign * np.asarray(pos, dtype=np.float64)[..., None] * inv
    zc = zc * np.exp(1j * ang)
    x[..., dim - rope_dim::2] = zc.real
    x[..., dim - rope_dim + 1::2] = zc.imag
    return x


def compress_masked(c: np.ndarray, z: np.ndarray, bias: np.ndarray, m: int, overlap: bool,
                    rope_dim: int = 0, theta: float = 10000.0, pos0: float = 0.0) -> np.ndarray:
    """Pooling as a masked softmax over the whole sequence axis.

    One sequence: c, z [S, dim] -> [S//m, dim].  A membership table gives, for
    every (entry, token), the token's offset inside the entry's window or -1."""
    c = np.asarray(c, np.float64)
    z = np.asarray(z, np.float64)
    S, dim = c.shape
    N = S // m
    s_idx = np.arange(N)[:, None]
    t_idx = np.arange(S)[None, :]
    start = (s_idx - 1) * m if overlap else s_idx * m
    width = 2 * m if overlap else m
    off = t_idx - start                                    # [N, S]
    member = (off >= 0) & (off < width)
    offc = np.clip(off, 0, width - 1)
    logits = z[None, :, :] + bias[offc]                    # [N, S, dim]
    logits = np.where(member[..., None], logits, -np.inf)
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    p = e / e.sum(axis=1, keepdims=True)
    pooled = np.einsum("nsd,sd->nd", p, c)
    if rope_dim:
        pooled = rope_complex(pooled, pos0 + np.arange(N) * m, rope_dim, theta, +1)
    return pooled


def sliding_causal_mask(S: int, W: int) -> np.ndarray:
    """[S, S] additive mask: 0 where t-W < j <= t, else -inf."""
    t = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    ok = (j <= t) & (j > t - W)
    return np.where(ok, 0.0, -np.inf)


def _eager(q_rot: np.ndarray, keys: np.ndarray, mask: np.ndarray, sinks, sm_scale: float) -> np.ndarray:
    """Eager attention with one shared K=V head and a per-head sink column.
    q_rot [S, H, D]; keys [S, K, D] (per-query key lists) or [K, D]; mask [S, K]."""
    if keys.ndim == 2:
        logits = np.einsum("thd,kd->thk", q_rot, keys) * sm_scale
    else:
        logits = np.einsum("thd,tkd->thk", q_rot, keys) * sm_scale
    logits = logits + mask[:, None, :]
    S, H = q_rot.shape[:2]
    if sinks is not None:
        sink_col = np.broadcast_to(np.asarray(sinks, np.float64)[None, :, None], (S, H, 1))
    else:
        sink_col = np.full((S, H, 1), -np.inf)
    full = np.concatenate([sink_col, logits], axis=-1)
    mx = full.max(axis=-1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.exp(full - mx)
    den = e.sum(axis=-1, keepdims=True)
    p = np.where(den > 0, e / np.where(den > 0, den, 1.0), 0.0)[..., 1:]   # the sink's value is zero
    if keys.ndim == 2:
        return np.einsum("thk,kd->thd", p, keys)
    return np.einsum("thk,tkd->thd", p, keys)


def csa_attention(q: np.ndarray, kv_rot: np.ndarray, pool: np.ndarray, idx: np.ndarray, sinks,
                  W: int, sm_scale: float, rope_dim: int, theta: float, pos0: float = 0.0) -> np.ndarray:
    """CSA layer, one sequence, HF flat-slot layout.

    q [S, H, D] unrotated; kv_rot [S, D] window K=V already rotated; pool [N, D]
    (rotated); idx [S, k] with -1 sentinels.  Keys are [kv_rot ; gathered S*k]
    and the mask is cat([sliding_causal_mask, block_bias], -1)."""
    S, H, D = q.shape
    k = idx.shape[1]
    pos = pos0 + np.arange(S)
    q_rot = rope_complex(q, pos[:, None], rope_dim, theta, +1)
    gathered = pool[np.clip(idx, 0, None)].reshape(S * k, D) if k else np.zeros((0, D))
    block_bias = np.full((S, S * k), -np.inf)
    for t in range(S):   # query t owns flat columns [t*k, (t+1)*k) after the S window columns
        block_bias[t, t * k:(t + 1) * k] = np.where(idx[t] >= 0, 0.0, -np.inf)
    mask = np.concatenate([sliding_causal_mask(S, W) if W > 0 else np.full((S, S), -np.inf),
                           block_bias], axis=-1)
    keys = np.concatenate([kv_rot, gathered], axis=0)
    o = _eager(q_rot, keys, mask, sinks, sm_scale)
    return rope_complex(o, pos[:, None], rope_dim, theta, -1)


def hca_attention(q: np.ndarray, kv_rot: np.ndarray, pool: np.ndarray, m: int, sinks,
                  W: int, sm_scale: float, rope_dim: int, theta: float, pos0: float = 0.0) -> np.ndarray:
    """HCA layer, one sequence: keys [kv_rot ; pool], block_bias lets query t see
    entry w iff w < (t+1)//m."""
    S, H, D = q.shape
    N = pool.shape[0]
    pos = pos0 + np.arange(S)
    q_rot = rope_complex(q, pos[:, None], rope_dim, theta, +1)
    w = np.arange(N)[None, :]
    t = np.arange(S)[:, None]
    block_bias = np.where(w < (t + 1) // m, 0.0, -np.inf)
    mask = np.concatenate([sliding_causal_mask(S, W) if W > 0 else np.full((S, S), -np.inf),
                           block_bias], axis=-1)
    keys = np.concatenate([kv_rot, pool], axis=0)
    o = _eager(q_rot, keys, mask, sinks, sm_scale)
    return rope_complex(o, pos[:, None], rope_dim, theta, -1)


def index_scores_dense(q_idx: np.ndarray, w: np.ndarray, kpool: np.ndarray, m: int,
                       scale: float) -> np.ndarray:
    """Indexer scores of one sequence as whole-matrix algebra with a causal
    block mask: [S, N] = scale * sum_h w[:, h] * relu(q_idx[:, h] @ kpool.T)."""
    S = q_idx.shape[0]
    N = kpool.shape[0]
    dots = np.einsum("thd,nd->thn", np.asarray(q_idx, np.float64), np.asarray(kpool, np.float64))
    sc = scale * np.einsum("th,thn->tn", np.asarray(w, np.float64), np.maximum(dots, 0.0))
    vis = np.arange(N)[None, :] < ((np.arange(S)[:, None] + 1) // m)
    return np.where(vis, sc, -np.inf)


def topk_by_sort(scores: np.ndarray, k: int) -> np.ndarray:
    """Top-k of each row by Python's sort on (-score, index); -inf entries are
    not candidates.  Output ascending, -1 fill."""
    out = np.full((scores.shape[0], k), -1, dtype=np.int32)
    for t, row in enumerate(scores):
        cand = [(-float(v), i) for i, v in enumerate(row) if np.isfinite(v)]
        pick = sorted(i for _, i in sorted(cand)[:k])
        out[t, :len(pick)] = pick
    return out
