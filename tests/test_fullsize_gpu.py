"""Parity at the full workload sizes, in the launch configuration bench.py times.

Each test builds the bench workload (same seeds, shapes and calls), runs one
step on the GPU, and checks sampled outputs against the oracle computed from
the same synthetic inputs (copied back to the host): the oracle recomputes the
whole chain itself (pool, index keys, rotated window, scores, top-k) and never
takes a value produced by the HIP path.  Attention outputs are compared on the
sampled rows whose top-k set equals the oracle's (rows with a near-tie at the
k-th score may legitimately differ; the gap rule checks those)."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from gpu_helpers import assert_close, check_topk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import dsv4_synth as S  # noqa: E402
import oracle as O  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


@pytest.fixture(scope="module")
def bench_mod(K):
    import bench
    return bench


def _b16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _f64rows(x, first_tok=None):
    x = np.ascontiguousarray(x, np.float64)
    return S.RowSet("f64", x.view(np.uint8).reshape(x.shape[0], x.shape[1], -1), x.shape[2],
                    np.full(x.shape[0], x.shape[1], np.int32),
                    first_tok=None if first_tok is None else np.asarray(first_tok, np.int32))


def _host_rows(rs, seqs, kind):
    """Device RowStore -> host RowSet of the sequences `seqs` (renumbered 0..)."""
    data = rs.data[seqs].contiguous()
    data = data.view(torch.uint8).cpu().numpy().reshape(len(seqs), rs.stride, -1)
    return S.RowSet(kind, data, rs.dim, rs.count[seqs].cpu().numpy().astype(np.int32), tail=rs.tail,
                    row_scale=None if rs.row_scale is None else rs.row_scale[seqs].cpu().numpy(),
                    blk_scale=None if rs.blk_scale is None else rs.blk_scale[seqs].cpu().numpy(),
                    first_tok=None if rs.first_tok is None else rs.first_tok[seqs].cpu().numpy().astype(np.int32))


def test_csa_prefill_S8192(K, bench_mod):
    """Flash-shaped CSA prefill, S=8192: pool, index keys, window rope (every
    row), top-k and attention on sampled query rows."""
    wl = bench_mod.CsaPrefill(torch, K, S)
    wl.step()
    torch.cuda.synchronize()
    Sx, m, R, th, D = wl.S, wl.m, wl.R, wl.theta, wl.D
    say("csa prefill S=8192: oracle pools")
    pool_o = O.compress(_b16(wl.c), _b16(wl.z), wl.bias.cpu().numpy(), m, True, R, th, np.zeros(1, np.int64),
                        kind="bf16")
    kpool_o = O.compress(_b16(wl.c_idx), _b16(wl.z_idx), wl.bias_idx.cpu().numpy(), m, True, kind="bf16")
    assert_close(wl.pool.float().cpu().numpy(), pool_o, "bf16", "pool")
    assert_close(wl.kpool.float().cpu().numpy(), kpool_o, "bf16", "index keys")
    kv = S.bf16_to_f32(_b16(wl.kv))
    kv_rot_o = O.rope(kv, np.arange(Sx), R, th, +1)
    assert_close(wl.kv_rot[0].float().cpu().numpy(), kv_rot_o, "bf16", "window rope")

    rng = np.random.default_rng(8192)
    rows = np.unique(np.concatenate([[0, 1, 3, 30, 31, 127, 128, 2046, 2047, 2048, 4095, 8190, 8191],
                                     rng.choice(Sx, 19, replace=False)])).astype(np.int32)
    seq = np.zeros(len(rows), np.int32)
    # the index keys are stored as bf16 (the storage type the chain asks for):
    # the oracle scores its own keys rounded the same way.  Its fp64 pooling and
    # the kernel's fp32 pooling can still round a few of the 262144 key values
    # to neighbouring bf16 codes, which moves those entries' scores by ~1e-3;
    # the gap rule here allows that much (the exact 1e-5 rule applies where
    # both sides score identical stored keys, in the decode cases below and in
    # the index parity tests).
    kp_rows = _f64rows(S.bf16_to_f32(S.bf16_bits(kpool_o.astype(np.float32))))
    sc = O.index_scores(seq, rows, _b16(wl.q_idx[rows]), "bf16", wl.w[rows].cpu().numpy(), kp_rows, m,
                        wl.score_scale)
    nv = O.n_visible(rows, m, Sx // m)
    idx_o = O.topk(sc, nv, wl.k)
    idx = wl.idx[rows].cpu().numpy()
    stats = check_topk(idx, sc, nv, wl.k, "csa prefill S=8192", gap=2e-3)
    say("top-k", stats)
    out_o = O.attn(seq, rows, np.zeros(1, np.int64), _b16(wl.q[rows]), "bf16", _f64rows(kv_rot_o[None], [0]), wl.W,
                   _f64rows(pool_o), "csa", idx=idx_o, sinks=wl.sinks.cpu().numpy(), sm_scale=wl.sm_scale,
                   rope_dim=R, theta=th)
    same = np.array([np.array_equal(np.sort(a[a >= 0]), np.sort(b[b >= 0])) for a, b in zip(idx, idx_o)])
    say("rows with the oracle's exact set", int(same.sum()), "of", len(rows))
    assert same.mean() >= 0.75
    assert_close(wl.out[rows].float().cpu().numpy()[same], out_o[same], "bf16", "csa attention S=8192")
    del wl
    torch.cuda.empty_cache()


def test_hca_prefill_S65536(K, bench_mod):
    """Flash-shaped HCA prefill, S=65536 (512 entries): pool (every entry) and
    attention on sampled query rows."""
    wl = bench_mod.HcaPrefill(torch, K, S)
    wl.step()
    torch.cuda.synchronize()
    Sx, m, R, th, W = wl.S, wl.m, wl.R, wl.theta, wl.W
    say("hca prefill S=65536: oracle pool")
    pool_o = O.compress(_b16(wl.c), _b16(wl.z), wl.bias.cpu().numpy(), m, False, R, th, np.zeros(1, np.int64),
                        kind="bf16")
    assert_close(wl.pool.float().cpu().numpy(), pool_o, "bf16", "hca pool")
    rng = np.random.default_rng(65536)
    rows = np.unique(np.concatenate([[0, 126, 127, 128, 255, 65535], rng.choice(Sx, 14, replace=False)])).astype(np.int32)
    # rotated window rows [t-W+1, t] of each sampled token, as a per-query window store
    lo = np.maximum(rows - W + 1, 0)
    win = np.zeros((len(rows), W, wl.D))
    for i, (a, t) in enumerate(zip(lo, rows)):
        kvb = S.bf16_to_f32(_b16(wl.kv[a:t + 1]))
        win[i, : t + 1 - a] = O.rope(kvb, np.arange(a, t + 1), R, th, +1)
    win_rows = _f64rows(win, lo)
    win_rows.count = (rows + 1 - lo).astype(np.int32)
    seq = np.arange(len(rows), dtype=np.int32)
    pool_rep = _f64rows(np.repeat(pool_o, len(rows), axis=0))
    out_o = O.attn(seq, rows, np.zeros(len(rows), np.int64), _b16(wl.q[rows]), "bf16", win_rows, W, pool_rep, "hca",
                   m=m, sinks=wl.sinks.cpu().numpy(), sm_scale=wl.sm_scale, rope_dim=R, theta=th)
    assert_close(wl.out[rows].float().cpu().numpy(), out_o, "bf16", "hca attention S=65536")
    del wl
    torch.cuda.empty_cache()


def test_csa_decode_B32_L131072(K, bench_mod):
    """CSA decode, 32 sequences x 131072 tokens: indexer top-k and FP8
    attention on sampled sequences."""
    wl = bench_mod.CsaDecode(torch, K, S, copies=1)
    wl.step()
    torch.cuda.synchronize()
    pool, win, kp, q, q_idx, w, sinks = wl.sets[0]
    seqs = [0, 13, 31]
    n = len(seqs)
    tok = np.full(n, wl.L - 1, np.int32)
    seq = np.arange(n, dtype=np.int32)
    say("csa decode: oracle scores over 32768 entries x", n)
    kp_h = _host_rows(kp, seqs, "bf16")
    sc = O.index_scores(seq, tok, _b16(q_idx[seqs]), "bf16", w[seqs].cpu().numpy(), kp_h, wl.m, wl.score_scale)
    nv = O.n_visible(tok, wl.m, kp_h.count)
    idx_o = O.topk(sc, nv, wl.k)
    idx = wl.idx[seqs].cpu().numpy()
    say("top-k", check_topk(idx, sc, nv, wl.k, "csa decode"))
    out_o = O.attn(seq, tok, np.zeros(n, np.int64), _b16(q[seqs]), "bf16", _host_rows(win, seqs, "fp8r"), wl.W,
                   _host_rows(pool, seqs, "fp8r"), "csa", idx=idx_o, sinks=sinks.cpu().numpy(), sm_scale=wl.sm_scale,
                   rope_dim=wl.R, theta=wl.theta)
    same = np.array([np.array_equal(np.sort(a[a >= 0]), np.sort(b[b >= 0])) for a, b in zip(idx, idx_o)])
    assert same.sum() >= n - 1
    assert_close(wl.out[seqs].float().cpu().numpy()[same], out_o[same], "bf16", "csa decode attention")
    del wl
    torch.cuda.empty_cache()


def test_mixed_decode_B8_L1048576(K, bench_mod):
    """1M-token mixed decode, 8 sequences: MXFP4 indexer top-k (262144 entries)
    with FP8 CSA attention, and dense FP8 HCA attention over 8192 entries."""
    wl = bench_mod.MixedDecode(torch, K, S, copies=1)
    wl.step()
    torch.cuda.synchronize()
    pool, win, kp, qpk, qsc, q, w, sinks, hpool, hwin, hq, hsinks = wl.sets[0]
    seqs = [2, 7]
    n = len(seqs)
    tok = np.full(n, wl.L - 1, np.int32)
    seq = np.arange(n, dtype=np.int32)
    say("mixed decode: oracle MXFP4 scores over 262144 entries x", n)
    kp_h = _host_rows(kp, seqs, "mxfp4")
    sc = O.index_scores(seq, tok, qpk[seqs].cpu().numpy(), "mxfp4", w[seqs].cpu().numpy(), kp_h, 4, wl.score_scale,
                        q_scale=qsc[seqs].cpu().numpy())
    nv = O.n_visible(tok, 4, kp_h.count)
    idx_o = O.topk(sc, nv, wl.k)
    idx = wl.idx[seqs].cpu().numpy()
    say("top-k", check_topk(idx, sc, nv, wl.k, "mixed decode"))
    out_o = O.attn(seq, tok, np.zeros(n, np.int64), _b16(q[seqs]), "bf16", _host_rows(win, seqs, "fp8r"), wl.W,
                   _host_rows(pool, seqs, "fp8r"), "csa", idx=idx_o, sinks=sinks.cpu().numpy(), sm_scale=wl.sm_scale,
                   rope_dim=wl.R, theta=wl.theta)
    same = np.array([np.array_equal(np.sort(a[a >= 0]), np.sort(b[b >= 0])) for a, b in zip(idx, idx_o)])
    assert same.sum() >= n - 1
    assert_close(wl.out[seqs].float().cpu().numpy()[same], out_o[same], "bf16", "mixed decode CSA attention")
    hout_o = O.attn(seq, tok, np.zeros(n, np.int64), _b16(hq[seqs]), "bf16", _host_rows(hwin, seqs, "fp8r"), wl.W,
                    _host_rows(hpool, seqs, "fp8r"), "hca", m=128, sinks=hsinks.cpu().numpy(), sm_scale=wl.sm_scale,
                    rope_dim=wl.R, theta=wl.theta)
    assert_close(wl.hout[seqs].float().cpu().numpy(), hout_o, "bf16", "mixed decode HCA attention")
    del wl
    torch.cuda.empty_cache()
