"""Edge cases of the attention calls on the GPU, against the oracle:

* the largest pick count the boundary takes (top-k 2048) on fp16 rows (a
  prefill-sized batch, one workgroup per query; and a few queries whose rows
  are split over workgroups) and on FP8 rows (decode);
* queries that see no row at all (no window, every pick -1, or an HCA token
  before its first pooled entry), with and without sinks: the output is zero
  (the sink's value vector is zero; with neither rows nor sink the softmax is
  empty and the library writes zeros).
"""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import assert_close, dev, tensor_of, upload_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


def _rows(rng, L, T, W, D, rows):
    """A pool of L / 4 entries, and window rows for tokens L - T - W + 1 .. L - 1:
    every one of the last T tokens finds its W window rows there."""
    N = L // 4
    tail = 64 if rows == "fp8r" else 0
    pool = S.rowset_from_values(rng.standard_normal((1, N, D)).astype(np.float32), rows, tail=tail)
    nw = T + W - 1
    win = S.rowset_from_values(rng.standard_normal((1, nw, D)).astype(np.float32), rows, count=np.full(1, nw),
                               first_tok=np.full(1, L - nw), tail=tail)
    return pool, win, N


@pytest.mark.parametrize("rows,T", [("f16", 600), ("f16", 4), ("fp8r", 4)])
def test_attn_topk_2048(K, rows, T):
    """Every query picks 2048 pool entries (the boundary's maximum) besides its
    128 window rows."""
    say("attention top-k 2048", rows, T)
    rng = np.random.default_rng(2048 + T)
    B, H, D, R, W, k, theta = 1, 64, 512, 64, 128, 2048, 1.6e5
    L = 4 * 2600
    pool, win, N = _rows(rng, L, T, W, D, rows)
    tok = np.arange(L - T, L, dtype=np.int32)
    seq = np.zeros(T, np.int32)
    q = S.bf16_to_f32(S.bf16_bits((1.28 * rng.standard_normal((T, H, D))).astype(np.float32)))
    nv = O.n_visible(tok, 4, np.full(T, N))
    idx = np.stack([np.sort(rng.choice(int(n), k, replace=False)) for n in nv]).astype(np.int32)
    sinks = rng.standard_normal(H).astype(np.float32)
    ref = O.attn(seq, tok, np.zeros(1, np.int64), S.bf16_bits(q), "bf16", win, W, pool, "csa", idx=idx, sinks=sinks,
                 sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    Q = K.QueryRows(dev(seq), dev(tok), dev(np.zeros(1, np.int64)), B)
    out = K.dsv4_sparse_attn(Q, tensor_of(q, "bf16"), upload_rows(win), W, upload_rows(pool), dev(idx), dev(sinks),
                             1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", f"top-k 2048, {rows} rows, {T} queries")


@pytest.mark.parametrize("rows,T,sink", [("f16", 520, False), ("f16", 520, True), ("f16", 3, False),
                                         ("fp8r", 3, False), ("fp8r", 3, True)])
def test_attn_queries_without_rows(K, rows, T, sink):
    """No window branch and every pick -1: nothing to attend to."""
    say("attention without rows", rows, T, sink)
    rng = np.random.default_rng(77 + T)
    B, H, D, R, theta = 1, 64, 512, 64, 1.6e5
    L = 4 * 600
    pool, _, N = _rows(rng, L, T, 128, D, rows)
    tok = np.arange(L - T, L, dtype=np.int32)
    seq = np.zeros(T, np.int32)
    q = S.bf16_to_f32(S.bf16_bits((1.28 * rng.standard_normal((T, H, D))).astype(np.float32)))
    idx = np.full((T, 16), -1, np.int32)
    sinks = rng.standard_normal(H).astype(np.float32) if sink else None
    ref = O.attn(seq, tok, np.zeros(1, np.int64), S.bf16_bits(q), "bf16", None, 0, pool, "csa", idx=idx, sinks=sinks,
                 sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    assert np.all(ref == 0.0)
    Q = K.QueryRows(dev(seq), dev(tok), dev(np.zeros(1, np.int64)), B)
    out = K.dsv4_sparse_attn(Q, tensor_of(q, "bf16"), None, 0, upload_rows(pool), dev(idx),
                             dev(sinks) if sink else None, 1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got)) and np.all(got == 0.0), f"{rows}: nonzero output for queries without rows"


@pytest.mark.parametrize("rows", ["f16", "bf16"])
def test_hca_tokens_before_the_first_entry(K, rows):
    """HCA with no window: tokens t < m' - 1 see no pooled entry; the rest see
    w < (t + 1) / m'.  A prefill-sized batch from token 0."""
    say("hca before the first entry", rows)
    rng = np.random.default_rng(128)
    B, H, D, R, m, theta = 1, 64, 512, 64, 128, 1.6e5
    Sx = 600
    N = Sx // m
    pool = S.rowset_from_values(rng.standard_normal((B, N, D)).astype(np.float32), rows)
    seq = np.zeros(Sx, np.int32)
    tok = np.arange(Sx, dtype=np.int32)
    q = S.bf16_to_f32(S.bf16_bits((1.28 * rng.standard_normal((Sx, H, D))).astype(np.float32)))
    sinks = rng.standard_normal(H).astype(np.float32)
    ref = O.attn(seq, tok, np.zeros(1, np.int64), S.bf16_bits(q), "bf16", None, 0, pool, "hca", m=m, sinks=sinks,
                 sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    assert np.all(ref[: m - 1] == 0.0)
    Q = K.QueryRows(dev(seq), dev(tok), dev(np.zeros(1, np.int64)), B)
    out = K.dsv4_hca_attn(Q, tensor_of(q, "bf16"), None, 0, upload_rows(pool), m, dev(sinks), 1 / np.sqrt(D), R,
                          theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[: m - 1] == 0.0)
    assert_close(got, ref, "bf16", f"hca without window, {rows} rows")
