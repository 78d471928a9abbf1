"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Sizes are chosen so the oracle finishes in seconds while every kernel still
runs several tiles and a ragged tail.  Inputs come from dsv4_synth; the oracle
never sees a value produced by the HIP path (where an attention test needs a
pool or an index set, both sides take the oracle's, rounded to the storage
type).
"""
import sys

import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import (assert_close, check_topk, dev, tensor_of, upload_rows)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


def f64rows(x, first_tok=None, count=None):
    x = np.asarray(x, np.float64)
    B, n, d = x.shape
    return S.RowSet("f64", x.copy().view(np.uint8).reshape(B, n, -1), d,
                    np.full(B, n, np.int32) if count is None else np.asarray(count, np.int32),
                    first_tok=None if first_tok is None else np.asarray(first_tok, np.int32))


# --------------------------------------------------------------------------- compressor / rope
@pytest.mark.parametrize("store,B,Sx,D,m,overlap,R,theta", [
    ("f32", 1, 256, 64, 4, True, 16, 1e4),
    ("bf16", 2, 700, 512, 4, True, 64, 1.6e5),
    ("bf16", 1, 1000, 512, 128, False, 64, 1.6e5),
    ("bf16", 2, 301, 128, 4, True, 0, 1.6e5),
    ("f32", 1, 37, 12, 1, False, 4, 100.0),
])
def test_compress(K, store, B, Sx, D, m, overlap, R, theta):
    say("compress", store, B, Sx, D, m, overlap, R)
    rng = np.random.default_rng(100 + Sx)
    round_ = (lambda x: S.bf16_to_f32(S.bf16_bits(x))) if store == "bf16" else (lambda x: x.astype(np.float32))
    c = round_(rng.standard_normal((B, Sx, D)).astype(np.float32) * 1.28)
    z = round_(rng.standard_normal((B, Sx, D)).astype(np.float32) * 1.28)
    width = 2 * m if overlap else m
    bias = (0.1 * rng.standard_normal((width, D))).astype(np.float32)
    pos0 = np.array([0, 12345][:B], np.int64)
    ref = O.compress(S.bf16_bits(c) if store == "bf16" else c, S.bf16_bits(z) if store == "bf16" else z,
                     bias, m, overlap, R, theta, pos0, kind=store)
    got = K.dsv4_compress(tensor_of(c, store), tensor_of(z, store), dev(bias), m, overlap, R, theta,
                          pos0=dev(pos0), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(got.cpu().numpy(), ref, store, "compress")
    # bf16 / fp16 outputs (every input type) round once more
    got16 = K.dsv4_compress(tensor_of(c, store), tensor_of(z, store), dev(bias), m, overlap, R, theta,
                            pos0=dev(pos0), out_dtype=torch.bfloat16)
    assert_close(got16.float().cpu().numpy(), ref, "bf16", "compress bf16 out")
    goth = K.dsv4_compress(tensor_of(c, store), tensor_of(z, store), dev(bias), m, overlap, R, theta,
                           pos0=dev(pos0), out_dtype=torch.float16)
    assert_close(goth.float().cpu().numpy(), ref, "bf16", "compress f16 out")


def test_compress_empty_and_short(K):
    say("compress empty")
    c = torch.zeros(1, 3, 8, device="cuda")
    out = K.dsv4_compress(c, c, torch.zeros(8, 8, device="cuda"), 4, True)
    assert out.shape == (1, 0, 8)


@pytest.mark.parametrize("store,D,R,theta", [("f32", 64, 16, 1e4), ("bf16", 512, 64, 1.6e5)])
def test_rope(K, store, D, R, theta):
    say("rope", store, D, R)
    rng = np.random.default_rng(7)
    n = 1000
    x = rng.standard_normal((n, D)).astype(np.float32)
    if store == "bf16":
        x = S.bf16_to_f32(S.bf16_bits(x))
    pos = rng.integers(0, 2 ** 20, n).astype(np.int64)
    pos[:3] = [0, 1, 2 ** 20 - 1]
    for inv in (False, True):
        ref = O.rope(x, pos, R, theta, -1 if inv else +1)
        got = K.dsv4_rope(tensor_of(x, store), dev(pos), R, theta, inverse=inv, out=None)
        torch.cuda.synchronize()
        tol_store = "f32" if store == "f32" else "bf16"
        assert_close(got.float().cpu().numpy(), ref, tol_store, f"rope inv={inv}")
        goth = K.dsv4_rope(tensor_of(x, store), dev(pos), R, theta, inverse=inv, out_dtype=torch.float16)
        assert_close(goth.float().cpu().numpy(), ref, "bf16", f"rope f16 out inv={inv}")
        if store == "f32":
            gotb = K.dsv4_rope(tensor_of(x, store), dev(pos), R, theta, inverse=inv, out_dtype=torch.bfloat16)
            assert_close(gotb.float().cpu().numpy(), ref, "bf16", f"rope bf16 out inv={inv}")


@pytest.mark.parametrize("store,D,R,n,offset", [
    ("f32", 6, 4, 70000, 0),      # a width that is not a multiple of 8, rows over two launches
    ("bf16", 30, 16, 1000, 0),
    ("bf16", 64, 64, 1000, 1),    # the input 2 bytes off 16-byte alignment
])
def test_rope_per_pair_path(K, store, D, R, n, offset):
    """Rows the eight-channel kernel does not take (width not a multiple of 8,
    or unaligned rows) go through the one-pair-per-thread kernel, whose launches
    hold at most 65535 rows each."""
    say("rope per-pair path", store, D, R, n, offset)
    rng = np.random.default_rng(9)
    theta = 1e4
    x = rng.standard_normal((n, D)).astype(np.float32)
    if store == "bf16":
        x = S.bf16_to_f32(S.bf16_bits(x))
    pos = rng.integers(0, 2 ** 20, n).astype(np.int64)
    xt = tensor_of(x, store)
    if offset:
        buf = torch.empty(n * D + offset, dtype=xt.dtype, device="cuda")
        view = buf[offset:offset + n * D].view(n, D)
        view.copy_(xt)
        xt = view
        assert xt.data_ptr() % 16 != 0
    for inv in (False, True):
        ref = O.rope(x, pos, R, theta, -1 if inv else +1)
        got = K.dsv4_rope(xt, dev(pos), R, theta, inverse=inv)
        torch.cuda.synchronize()
        assert_close(got.float().cpu().numpy(), ref, "f32" if store == "f32" else "bf16", f"rope inv={inv}")


# --------------------------------------------------------------------------- indexer + top-k
def _prefill_indexer_case(store, B, Sx, Hi, Di, m, k, seed):
    rng = np.random.default_rng(seed)
    rnd = (lambda x: S.bf16_to_f32(S.bf16_bits(x))) if store == "bf16" else (lambda x: x.astype(np.float32))
    N = Sx // m
    keys = rnd(rng.standard_normal((B, N, Di)).astype(np.float32))
    q_idx = rnd(1.28 * rng.standard_normal((B * Sx, Hi, Di)).astype(np.float32))
    w = (1.28 * rng.standard_normal((B * Sx, Hi))).astype(np.float32)
    seq = np.repeat(np.arange(B), Sx).astype(np.int32)
    tok = np.tile(np.arange(Sx), B).astype(np.int32)
    return keys, q_idx, w, seq, tok


@pytest.mark.parametrize("store,B,Sx,Hi,Di,m,k", [
    ("f32", 1, 256, 4, 32, 4, 8),
    ("bf16", 2, 700, 64, 128, 4, 64),
    ("bf16", 1, 300, 16, 64, 4, 8),
    ("bf16", 1, 2050, 64, 128, 4, 512),
    ("bf16", 3, 701, 64, 128, 4, 64),    # 4-query groups straddle sequences
    ("bf16", 2, 1030, 32, 128, 4, 100),
    ("bf16", 1, 6000, 64, 128, 4, 512),  # pools of 1025..1500 entries: the 2048-entry select
])
def test_index_topk_prefill(K, store, B, Sx, Hi, Di, m, k):
    say("index_topk prefill", store, B, Sx, Hi, Di, m, k)
    keys, q_idx, w, seq, tok = _prefill_indexer_case(store, B, Sx, Hi, Di, m, k, 11 + Sx)
    kind = store
    kp = S.rowset_from_values(keys, kind)
    scale = 1.0 / np.sqrt(Hi * Di)
    qstore = S.bf16_bits(q_idx) if store == "bf16" else q_idx
    ref = O.index_scores(seq, tok, qstore, kind, w, kp, m, scale)
    nv = O.n_visible(tok, m, kp.count[seq])
    Q = K.QueryRows(dev(seq), dev(tok), None, B)
    idx, sc = K.dsv4_index_topk(Q, tensor_of(q_idx, store), dev(w), upload_rows(kp), m, k, scale, want_scores=True)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    stats = check_topk(idx, ref, nv, k, "prefill")
    say("topk stats", stats)
    # the reported scores of the picks match the oracle's within fp32 accumulation error
    sc = sc.cpu().numpy()
    for r in range(0, idx.shape[0], 37):
        p = idx[r][idx[r] >= 0]
        assert np.allclose(sc[r, :len(p)], ref[r, p], rtol=1e-4, atol=1e-5)


@pytest.mark.parametrize("B,Sx,k", [
    (1, 2050, 512),   # every row takes all its visible entries
    (3, 701, 64),     # 4-query groups straddle sequences; rows on both sides of n = k
    (1, 6000, 512),   # the 2048-entry select next to rows that are not scored
])
def test_index_topk_prefill_without_scores(K, B, Sx, k):
    """Without pick scores, rows with at most k visible entries are not scored:
    their picks are all of them.  The picks equal those of the call that
    returns scores, and the oracle's under the gap rule."""
    say("index_topk prefill, no scores", B, Sx, k)
    Hi, Di, m = 64, 128, 4
    keys, q_idx, w, seq, tok = _prefill_indexer_case("bf16", B, Sx, Hi, Di, m, k, 11 + Sx)
    kp = S.rowset_from_values(keys, "bf16")
    scale = 1.0 / np.sqrt(Hi * Di)
    ref = O.index_scores(seq, tok, S.bf16_bits(q_idx), "bf16", w, kp, m, scale)
    nv = O.n_visible(tok, m, kp.count[seq])
    Q = K.QueryRows(dev(seq), dev(tok), None, B)
    kpd = upload_rows(kp)
    qd = tensor_of(q_idx, "bf16")
    idx_s, _ = K.dsv4_index_topk(Q, qd, dev(w), kpd, m, k, scale, want_scores=True)
    idx_n = K.dsv4_index_topk(Q, qd, dev(w), kpd, m, k, scale)
    torch.cuda.synchronize()
    idx_s, idx_n = idx_s.cpu().numpy(), idx_n.cpu().numpy()
    assert np.array_equal(idx_n, idx_s)
    short = nv <= k
    assert short.any()
    for r in np.nonzero(short)[0]:
        assert np.array_equal(idx_n[r, :nv[r]], np.arange(nv[r])) and (idx_n[r, nv[r]:] == -1).all()
    check_topk(idx_n, ref, nv, k, "prefill, no scores")


@pytest.mark.parametrize("kind,B,L,k,Hi,Di", [
    ("bf16", 3, [1000, 40001, 20050], 512, 64, 128),
    ("mxfp4", 2, [70000, 5003], 1024, 64, 128),
    ("bf16", 2, [20000, 9], 2048, 64, 128),
    ("mxfp4", 1, [4 * 16384 + 7], 1, 64, 128),
    # rows longer than one workgroup's select: the radix-threshold passes over
    # 4096-entry chunks, next to rows that take every entry or have none
    ("bf16", 3, [4 * 20000, 4 * 300, 3], 2048, 64, 128),
    ("bf16", 1, [4 * 200000], 2048, 64, 128),
    # the other indexer head counts and head dims of the scan
    ("mxfp4", 2, [30000, 4001], 512, 16, 128),
    ("mxfp4", 2, [30000, 4001], 512, 48, 128),
    ("bf16", 2, [30000, 4001], 512, 32, 96),
    ("bf16", 2, [30000, 4001], 512, 48, 32),
    ("bf16", 2, [4 * 3000 + 1, 4 * 2100], 512, 64, 128),   # rows of 2049..4096 entries: 16 keys per thread
    ("f32", 1, [4 * 20000], 512, 4, 32),   # fp32 scores of a long row: the level-0 histogram in its own pass
])
def test_index_topk_decode(K, kind, B, L, k, Hi, Di):
    say("index_topk decode", kind, B, L, k, Hi, Di)
    layer = S.decode_layer(31 + B, "csa", B, L, topk=k, idx_kind=kind, Hi=Hi, Di=Di)
    kp = layer.kpool
    tok = layer.tok
    seq = np.arange(B, dtype=np.int32)
    if kind == "mxfp4":
        qst, qsc = layer.q_idx_packed, layer.q_idx_scale
        qdev, qscd = dev(qst), dev(qsc)
    else:
        qst, qsc = (S.bf16_bits(layer.q_idx) if kind == "bf16" else layer.q_idx), None
        qdev, qscd = tensor_of(layer.q_idx, kind), None
    ref = O.index_scores(seq, tok, qst, kind, layer.w_idx, kp, layer.m, layer.score_scale, q_scale=qsc)
    nv = O.n_visible(tok, layer.m, kp.count)
    Q = K.QueryRows(dev(seq), dev(tok), None, B)
    idx, sc = K.dsv4_index_topk(Q, qdev, dev(layer.w_idx), upload_rows(kp), layer.m, k, layer.score_scale,
                                q_idx_scale=qscd, want_scores=True)
    torch.cuda.synchronize()
    idx, sc = idx.cpu().numpy(), sc.cpu().numpy()
    stats = check_topk(idx, ref, nv, k, "decode")
    say("topk stats", stats)
    for r in range(B):   # picks in ascending entry order, each with its score
        p = idx[r][idx[r] >= 0]
        assert np.all(np.diff(p) > 0), f"row {r}: picks not in ascending order"
        assert np.allclose(sc[r, :len(p)], ref[r, p], rtol=1e-4, atol=1e-5), f"row {r}: pick scores"
        assert np.all(np.isneginf(sc[r, len(p):])), f"row {r}: scores past the picks"


@pytest.mark.parametrize("B,L,k,n_distinct", [
    (2, [4 * 30000, 4 * 3000 + 3], 512, 3),   # radix-threshold passes over several chunks
    (1, [4 * 20000], 1024, 1),                # every score equal
    (3, [4 * 5000, 4 * 700, 9], 256, 2),      # one workgroup per row
    (3, [4 * 2000, 4 * 700 + 3, 9], 512, 3),  # 128-thread workgroups (pools of at most 2048)
    (2, [4 * 2048, 4 * 1500], 1024, 1),       # 128-thread workgroups, every score equal
])
def test_index_topk_ties(K, B, L, k, n_distinct):
    """Pool rows repeat a few distinct keys in runs of 7, so each row's scores
    take n_distinct values with thousands of exact ties: the picks must be the
    oracle's exactly (ties to the lower entry)."""
    say("index_topk ties", B, L, k, n_distinct)
    layer = S.decode_layer(77 + B, "csa", B, L, topk=k)
    kp = layer.kpool
    rows = kp.data.view(np.uint16).reshape(B, kp.rows_per_seq, -1)
    pick = (np.arange(kp.rows_per_seq) // 7) % n_distinct
    rows[:] = rows[:, pick, :]
    seq = np.arange(B, dtype=np.int32)
    tok = layer.tok
    qst = S.bf16_bits(layer.q_idx)
    ref = O.index_scores(seq, tok, qst, "bf16", layer.w_idx, kp, layer.m, layer.score_scale)
    nv = O.n_visible(tok, layer.m, kp.count)
    want = O.topk(ref, nv, k)
    Q = K.QueryRows(dev(seq), dev(tok), None, B)
    idx = K.dsv4_index_topk(Q, tensor_of(layer.q_idx, "bf16"), dev(layer.w_idx), upload_rows(kp), layer.m, k,
                            layer.score_scale)
    torch.cuda.synchronize()
    idx = idx.cpu().numpy()
    for r in range(B):
        assert np.array_equal(np.sort(idx[r][idx[r] >= 0]), np.sort(want[r][want[r] >= 0])), f"row {r}"
        assert np.array_equal(idx[r] >= 0, want[r] >= 0), f"row {r}: sentinel layout"
        p = idx[r][idx[r] >= 0]
        assert np.all(np.diff(p) > 0), f"row {r}: picks not in ascending order"


# --------------------------------------------------------------------------- attention
def _attn_prefill_inputs(B, Sx, H, D, R, W, m, theta, seed, overlap=True, rows="bf16"):
    """q values rounded to bf16; window rows rotated by the oracle; rows stored
    as `rows` ('bf16' or 'f16')."""
    rng = np.random.default_rng(seed)
    r16 = lambda x: S.bf16_to_f32(S.bf16_bits(x.astype(np.float32)))
    q = r16(1.28 * rng.standard_normal((B, Sx, H, D)))
    kv = 1.28 * rng.standard_normal((B, Sx, D))
    pos0 = np.array([0, 777, 5][:B], np.int64)
    kv_rot = np.stack([O.rope(kv[b], pos0[b] + np.arange(Sx), R, theta, +1) for b in range(B)])
    win = S.rowset_from_values(kv_rot.astype(np.float32), rows, count=np.full(B, Sx), first_tok=np.zeros(B))
    N = Sx // m
    pool_vals = (1.28 * rng.standard_normal((B, N, D))).astype(np.float32)
    pool = S.rowset_from_values(pool_vals, rows)
    sinks = rng.standard_normal(H).astype(np.float32)
    return q, win, pool, sinks, pos0


@pytest.mark.parametrize("B,Sx,H,W,m,k,rows", [
    (2, 520, 64, 128, 4, 64, "bf16"),
    (1, 300, 16, 40, 4, 200, "bf16"),   # k >= n: every visible entry
    (1, 200, 32, 0, 4, 16, "bf16"),     # no window branch
    (2, 520, 64, 128, 4, 64, "f16"),
    (1, 300, 16, 40, 4, 200, "f16"),
    (1, 200, 32, 0, 4, 16, "f16"),
    (1, 700, 48, 128, 4, 100, "f16"),
])
def test_sparse_attn_prefill(K, B, Sx, H, W, m, k, rows):
    say("sparse_attn prefill", B, Sx, H, W, m, k, rows)
    D, R, theta = 512, 64, 1.6e5
    q, win, pool, sinks, pos0 = _attn_prefill_inputs(B, Sx, H, D, R, W, m, theta, 40 + Sx, rows=rows)
    rng = np.random.default_rng(3)
    N = Sx // m
    seq = np.repeat(np.arange(B), Sx).astype(np.int32)
    tok = np.tile(np.arange(Sx), B).astype(np.int32)
    nv = O.n_visible(tok, m, np.full(len(tok), N))
    sc = rng.standard_normal((B * Sx, N))
    idx = O.topk(np.where(np.arange(N)[None] < nv[:, None], sc, -np.inf), nv, k)
    qs = S.bf16_bits(q.reshape(B * Sx, H, D))
    ref = O.attn(seq, tok, pos0, qs, "bf16", win if W else None, W, pool, "csa", idx=idx, sinks=sinks,
                 sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    Q = K.QueryRows(dev(seq), dev(tok), dev(pos0), B)
    out = K.dsv4_sparse_attn(Q, tensor_of(q.reshape(B * Sx, H, D), "bf16"), upload_rows(win) if W else None, W,
                             upload_rows(pool), dev(idx), dev(sinks), 1 / np.sqrt(D), R, theta,
                             out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", "sparse_attn")


@pytest.mark.parametrize("B,R,out", [
    (1, 64, "bf16"),    # bf16 outputs staged as whole head rows
    (2, 32, "bf16"),    # fewer rotated channels: the inverse rotation in one or two waves' blocks
    (1, 0, "bf16"),     # no rotated channels
    (1, 16, "f32"),
])
def test_sparse_attn_prefill_rope_out(K, B, R, out):
    """The fp16-row kernel's epilogue with every output-channel split of the rotated channels."""
    say("sparse_attn prefill rope/out", B, R, out)
    Sx, H, W, m, k, D, theta = 400, 64, 128, 4, 64, 512, 1.6e5
    q, win, pool, sinks, pos0 = _attn_prefill_inputs(B, Sx, H, D, R, W, m, theta, 60 + R, rows="f16")
    rng = np.random.default_rng(5)
    N = Sx // m
    seq = np.repeat(np.arange(B), Sx).astype(np.int32)
    tok = np.tile(np.arange(Sx), B).astype(np.int32)
    nv = O.n_visible(tok, m, np.full(len(tok), N))
    sc = rng.standard_normal((B * Sx, N))
    idx = O.topk(np.where(np.arange(N)[None] < nv[:, None], sc, -np.inf), nv, k)
    qs = S.bf16_bits(q.reshape(B * Sx, H, D))
    ref = O.attn(seq, tok, pos0, qs, "bf16", win, W, pool, "csa", idx=idx, sinks=sinks,
                 sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    Q = K.QueryRows(dev(seq), dev(tok), dev(pos0), B)
    got = K.dsv4_sparse_attn(Q, tensor_of(q.reshape(B * Sx, H, D), "bf16"), upload_rows(win), W,
                             upload_rows(pool), dev(idx), dev(sinks), 1 / np.sqrt(D), R, theta,
                             out_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    assert_close(got.float().cpu().numpy(), ref, "bf16", f"sparse_attn R={R} out={out}")


@pytest.mark.parametrize("H,rows", [(16, "f16"), (32, "f16"), (48, "f16"), (16, "fp8r"), (32, "fp8r"), (48, "fp8r")])
def test_attn_rope32_every_head_count(K, H, rows):
    """Each head count's kernel instance with a rope width other than 64 (a
    run-time width): fp16 prefill rows and FP8 decode rows (64 bf16 tail
    channels, the last 32 of them rotated)."""
    say("attention rope 32", H, rows)
    D, R, theta = 512, 32, 1.6e5
    if rows == "f16":
        B, Sx, W, m, k = 1, 300, 128, 4, 64
        q, win, pool, sinks, pos0 = _attn_prefill_inputs(B, Sx, H, D, R, W, m, theta, 80 + H, rows="f16")
        rng = np.random.default_rng(81)
        N = Sx // m
        seq = np.zeros(Sx, np.int32)
        tok = np.arange(Sx, dtype=np.int32)
        nv = O.n_visible(tok, m, np.full(Sx, N))
        idx = O.topk(np.where(np.arange(N)[None] < nv[:, None], rng.standard_normal((Sx, N)), -np.inf), nv, k)
        qs = S.bf16_bits(q.reshape(Sx, H, D))
        ref = O.attn(seq, tok, pos0, qs, "bf16", win, W, pool, "csa", idx=idx, sinks=sinks,
                     sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
        Q = K.QueryRows(dev(seq), dev(tok), dev(pos0), B)
        out = K.dsv4_sparse_attn(Q, tensor_of(q.reshape(Sx, H, D), "bf16"), upload_rows(win), W, upload_rows(pool),
                                 dev(idx), dev(sinks), 1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
    else:
        B, L, k = 2, [5000, 2222], 256
        layer = S.decode_layer(82 + H, "csa", B, L, H=H, R=R, topk=k, tail=64)
        seq = np.arange(B, dtype=np.int32)
        rng = np.random.default_rng(83)
        nv = O.n_visible(layer.tok, layer.m, layer.pool.count)
        sc = rng.standard_normal((B, layer.pool.rows_per_seq))
        idx = O.topk(np.where(np.arange(sc.shape[1])[None] < nv[:, None], sc, -np.inf), nv, k)
        ref = O.attn(seq, layer.tok, layer.pos0, S.bf16_bits(layer.q), "bf16", layer.win, layer.W, layer.pool, "csa",
                     idx=idx, sinks=layer.sinks, sm_scale=layer.sm_scale, rope_dim=R, theta=layer.theta)
        Q = K.QueryRows(dev(seq), dev(layer.tok), dev(layer.pos0), B)
        out = K.dsv4_sparse_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(layer.win), layer.W,
                                 upload_rows(layer.pool), dev(idx), dev(layer.sinks), layer.sm_scale, R, layer.theta,
                                 out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", f"attention rope 32, {H} heads, {rows} rows")


@pytest.mark.parametrize("B,Sx,H,W,m,sink,rows", [
    (1, 1100, 64, 128, 16, True, "bf16"),
    (2, 300, 64, 128, 128, True, "bf16"),
    (1, 150, 16, 0, 1, True, "bf16"),      # m' = 1, no window: causal MQA with sink
    (1, 90, 16, 7, 8, False, "bf16"),
    (1, 1100, 64, 128, 16, True, "f16"),
    (2, 300, 64, 128, 128, True, "f16"),
    (1, 150, 16, 0, 1, True, "f16"),
    (1, 90, 32, 7, 8, False, "f16"),
])
def test_hca_attn_prefill(K, B, Sx, H, W, m, sink, rows):
    say("hca_attn prefill", B, Sx, H, W, m, sink, rows)
    D, R, theta = 512, 64, 1.6e5
    q, win, pool, sinks, pos0 = _attn_prefill_inputs(B, Sx, H, D, R, W, m, theta, 50 + Sx, rows=rows)
    seq = np.repeat(np.arange(B), Sx).astype(np.int32)
    tok = np.tile(np.arange(Sx), B).astype(np.int32)
    qs = S.bf16_bits(q.reshape(B * Sx, H, D))
    ref = O.attn(seq, tok, pos0, qs, "bf16", win if W else None, W, pool, "hca", m=m,
                 sinks=sinks if sink else None, sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    Q = K.QueryRows(dev(seq), dev(tok), dev(pos0), B)
    out = K.dsv4_hca_attn(Q, tensor_of(q.reshape(B * Sx, H, D), "bf16"), upload_rows(win) if W else None, W,
                          upload_rows(pool), m, dev(sinks) if sink else None, 1 / np.sqrt(D), R, theta,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", "hca_attn")


@pytest.mark.parametrize("kind,B,L,k,H,tail", [
    ("csa", 3, [1000, 4093, 2050], 256, 64, 64),
    ("csa", 2, [131072, 700], 512, 64, 64),
    ("csa", 2, [9000, 37], 512, 16, 64),      # 16 heads; a sequence shorter than the window
    ("csa", 2, [5000, 2222], 256, 32, 32),    # 32 bf16 tail channels: the generic FP8 kernel
    ("hca", 2, [70000, 3000], 0, 64, 64),
    ("hca", 1, [3000], 0, 32, 64),           # 32 heads: two waves on the channel-split path
    ("hca", 1, [100], 0, 48, 64),
])
def test_attn_decode_fp8(K, kind, B, L, k, H, tail):
    say("attn decode fp8", kind, B, L, k, H, tail)
    layer = S.decode_layer(60 + B, kind, B, L, H=H, topk=max(k, 1), tail=tail)
    seq = np.arange(B, dtype=np.int32)
    tok = layer.tok
    qs = S.bf16_bits(layer.q)
    Q = K.QueryRows(dev(seq), dev(tok), dev(layer.pos0), B)
    if kind == "csa":
        rng = np.random.default_rng(5)
        N = layer.pool.count
        sc = rng.standard_normal((B, layer.pool.rows_per_seq))
        nv = O.n_visible(tok, layer.m, N)
        idx = O.topk(np.where(np.arange(sc.shape[1])[None] < nv[:, None], sc, -np.inf), nv, k)
        ref = O.attn(seq, tok, layer.pos0, qs, "bf16", layer.win, layer.W, layer.pool, "csa", idx=idx,
                     sinks=layer.sinks, sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
        out = K.dsv4_sparse_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(layer.win), layer.W,
                                 upload_rows(layer.pool), dev(idx), dev(layer.sinks), layer.sm_scale, layer.R,
                                 layer.theta, out_dtype=torch.float32)
    else:
        ref = O.attn(seq, tok, layer.pos0, qs, "bf16", layer.win, layer.W, layer.pool, "hca", m=layer.m,
                     sinks=layer.sinks, sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
        out = K.dsv4_hca_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(layer.win), layer.W,
                              upload_rows(layer.pool), layer.m, dev(layer.sinks), layer.sm_scale, layer.R,
                              layer.theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", f"{kind} decode")


@pytest.mark.parametrize("kind,B,L,k,H", [
    ("csa", 2, [20000, 3001], 256, 64),
    ("hca", 2, [70000, 3000], 0, 32),
    ("csa", 1, [5000], 128, 16),
])
def test_attn_decode_f16_split(K, kind, B, L, k, H):
    """fp16 K=V rows at decode shapes: a few query rows over long row lists, so
    each query's rows are split over several workgroups on the channel-split PV
    path (partials of every wave's channel slice) and merged by k_attn_combine."""
    say("attn decode f16 split", kind, B, L, k, H)
    layer = S.decode_layer(70 + B, kind, B, L, H=H, topk=max(k, 1))
    rng = np.random.default_rng(71)
    D = layer.D
    pool = S.rowset_from_values(rng.standard_normal((B, layer.pool.rows_per_seq, D)).astype(np.float32), "f16",
                                count=layer.pool.count)
    win = S.rowset_from_values(rng.standard_normal((B, layer.W, D)).astype(np.float32), "f16",
                               count=layer.win.count, first_tok=layer.win.first_tok)
    seq = np.arange(B, dtype=np.int32)
    tok = layer.tok
    qs = S.bf16_bits(layer.q)
    Q = K.QueryRows(dev(seq), dev(tok), dev(layer.pos0), B)
    if kind == "csa":
        N = pool.count
        sc = rng.standard_normal((B, pool.rows_per_seq))
        nv = O.n_visible(tok, layer.m, N)
        idx = O.topk(np.where(np.arange(sc.shape[1])[None] < nv[:, None], sc, -np.inf), nv, k)
        ref = O.attn(seq, tok, layer.pos0, qs, "bf16", win, layer.W, pool, "csa", idx=idx, sinks=layer.sinks,
                     sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
        out = K.dsv4_sparse_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(win), layer.W, upload_rows(pool),
                                 dev(idx), dev(layer.sinks), layer.sm_scale, layer.R, layer.theta,
                                 out_dtype=torch.float32)
    else:
        ref = O.attn(seq, tok, layer.pos0, qs, "bf16", win, layer.W, pool, "hca", m=layer.m, sinks=layer.sinks,
                     sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
        out = K.dsv4_hca_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(win), layer.W, upload_rows(pool),
                              layer.m, dev(layer.sinks), layer.sm_scale, layer.R, layer.theta,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", f"{kind} decode, fp16 rows")


# --------------------------------------------------------------------------- end to end
def test_tiny_csa_layer_end_to_end(K):
    """The tiny fp32 CSA layer (seq 256, 8 heads x 64, m=4, window 16, indexer
    4 x 32, top-k 8): every step on the GPU against the oracle chain."""
    say("tiny layer fp32")
    c = S.tiny_csa_layer()
    B, Sx, H, D, R, m, W, k = c.B, c.S, c.H, c.D, c.R, c.m, c.W, c.topk
    pos0 = c.pos0
    # oracle chain
    pool_o = O.compress(c.c, c.z, c.bias, m, True, R, c.theta, pos0)
    kpool_o = O.compress(c.c_idx, c.z_idx, c.bias_idx, m, True)
    kv_rot_o = O.rope(c.kv[0], pos0[0] + np.arange(Sx), R, c.theta, +1)[None]
    seq = np.zeros(Sx, np.int32)
    tok = np.arange(Sx, dtype=np.int32)
    sc_o = O.index_scores(seq, tok, c.q_idx[0], "f32", c.w_idx[0], f64rows(kpool_o), m, c.score_scale)
    nv = O.n_visible(tok, m, Sx // m)
    idx_o = O.topk(sc_o, nv, k)
    out_o = O.attn(seq, tok, pos0, c.q[0], "f32", f64rows(kv_rot_o, first_tok=[0]), W, f64rows(pool_o), "csa",
                   idx=idx_o, sinks=c.sinks, sm_scale=c.sm_scale, rope_dim=R, theta=c.theta)
    # HIP chain
    Q = K.QueryRows(dev(seq), dev(tok), dev(pos0), B)
    pool = K.dsv4_compress(dev(c.c), dev(c.z), dev(c.bias), m, True, R, c.theta, pos0=dev(pos0))
    kpool = K.dsv4_compress(dev(c.c_idx), dev(c.z_idx), dev(c.bias_idx), m, True)
    kv_rot = K.dsv4_rope(dev(c.kv[0]), dev(pos0[0] + np.arange(Sx)), R, c.theta)
    cnt = dev(np.full(1, Sx // m, np.int32))
    kps = K.RowStore(kpool, K.DSV4_F32, c.Di, cnt)
    idx = K.dsv4_index_topk(Q, dev(c.q_idx[0]), dev(c.w_idx[0]), kps, m, k, c.score_scale)
    win = K.RowStore(kv_rot[None].contiguous(), K.DSV4_F32, D, dev(np.full(1, Sx, np.int32)),
                     first_tok=dev(np.zeros(1, np.int32)))
    out = K.dsv4_sparse_attn(Q, dev(c.q[0]), win, W, K.RowStore(pool, K.DSV4_F32, D, cnt), idx, dev(c.sinks),
                             c.sm_scale, R, c.theta)
    torch.cuda.synchronize()
    assert_close(pool.cpu().numpy(), pool_o, "f32", "pool")
    assert_close(kpool.cpu().numpy(), kpool_o, "f32", "index keys")
    assert_close(kv_rot.cpu().numpy(), kv_rot_o[0], "f32", "window rope")
    idx = idx.cpu().numpy()
    stats = check_topk(idx, sc_o, nv, k, "tiny")
    say("tiny topk", stats)
    # the chain's output where its picks are the oracle's; every row with the
    # oracle's picks (exact ties of ReLU-zero scores may resolve either way)
    same = np.all(np.sort(np.where(idx < 0, 1 << 30, idx), 1) == np.sort(np.where(idx_o < 0, 1 << 30, idx_o), 1), 1)
    assert_close(out.cpu().numpy()[same], out_o[same], "f32", "tiny attention (chain)")
    out2 = K.dsv4_sparse_attn(Q, dev(c.q[0]), win, W, K.RowStore(pool, K.DSV4_F32, D, cnt), dev(idx_o), dev(c.sinks),
                              c.sm_scale, R, c.theta)
    torch.cuda.synchronize()
    assert_close(out2.cpu().numpy(), out_o, "f32", "tiny attention")


def test_csa_layer_bf16_end_to_end(K):
    """Flash-shaped CSA prefill at S=700 (B=2): compress + rope + indexer + top-k
    + sparse attention, all on the GPU, against the oracle chain."""
    say("csa layer bf16 S=700")
    c = S.flash_prefill(1234, "csa", B=2, S=700, topk=64, pos0=[0, 3000])
    B, Sx, H, D, R, m, W, k = c.B, c.S, c.H, c.D, c.R, c.m, c.W, c.topk
    b16 = S.bf16_bits
    pool_o = O.compress(b16(c.c), b16(c.z), c.bias, m, True, R, c.theta, c.pos0, kind="bf16")
    kpool_o = O.compress(b16(c.c_idx), b16(c.z_idx), c.bias_idx, m, True, kind="bf16")
    kv_rot_o = np.stack([O.rope(c.kv[b], c.pos0[b] + np.arange(Sx), R, c.theta, +1) for b in range(B)])
    seq = np.repeat(np.arange(B), Sx).astype(np.int32)
    tok = np.tile(np.arange(Sx), B).astype(np.int32)
    q_idx = c.q_idx.reshape(B * Sx, c.Hi, c.Di)
    w = c.w_idx.reshape(B * Sx, c.Hi)
    nv = O.n_visible(tok, m, np.full(len(tok), Sx // m))
    qv = c.q.reshape(B * Sx, H, D)
    # HIP chain
    Q = K.QueryRows(dev(seq), dev(tok), dev(c.pos0), B)
    pool = K.dsv4_compress(tensor_of(c.c, "bf16"), tensor_of(c.z, "bf16"), dev(c.bias), m, True, R, c.theta,
                           pos0=dev(c.pos0))
    kpool = K.dsv4_compress(tensor_of(c.c_idx, "bf16"), tensor_of(c.z_idx, "bf16"), dev(c.bias_idx), m, True)
    pos = dev((c.pos0[:, None] + np.arange(Sx)[None]).reshape(-1).astype(np.int64))
    kv_rot = K.dsv4_rope(tensor_of(c.kv.reshape(B * Sx, D), "bf16"), pos, R, c.theta)
    cnt = dev(np.full(B, Sx // m, np.int32))
    idx = K.dsv4_index_topk(Q, tensor_of(q_idx, "bf16"), dev(w), K.RowStore(kpool, K.DSV4_BF16, c.Di, cnt), m, k,
                            c.score_scale)
    win = K.RowStore(kv_rot.view(B, Sx, D), K.DSV4_BF16, D, dev(np.full(B, Sx, np.int32)),
                     first_tok=dev(np.zeros(B, np.int32)))
    out = K.dsv4_sparse_attn(Q, tensor_of(qv, "bf16"), win, W, K.RowStore(pool, K.DSV4_BF16, D, cnt), idx,
                             dev(c.sinks), c.sm_scale, R, c.theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert_close(pool.float().cpu().numpy(), pool_o, "bf16", "pool")
    # top-k on shared stored keys (the oracle's pooled keys as bf16, scored by
    # both sides): the 1e-5 gap rule
    kp_store = S.rowset_from_values(kpool_o.astype(np.float32), "bf16")
    sc_s = O.index_scores(seq, tok, b16(q_idx), "bf16", w, kp_store, m, c.score_scale)
    idx_s = K.dsv4_index_topk(Q, tensor_of(q_idx, "bf16"), dev(w), upload_rows(kp_store), m, k, c.score_scale)
    torch.cuda.synchronize()
    say("shared-key topk", check_topk(idx_s.cpu().numpy(), sc_s, nv, k, "csa layer S=700 (shared keys)"))
    idx_o = O.topk(sc_s, nv, k)
    # the chain's own picks over the GPU-pooled keys: counts, ranges, sentinel
    # layout, and the end-to-end gap bound for keys pooled in fp32 vs fp64
    say("chain topk", check_topk(idx.cpu().numpy(), sc_s, nv, k, "csa layer S=700 chain", gap=2e-3))
    # attention on the GPU-made pool and window with the oracle's picks: every row
    out = K.dsv4_sparse_attn(Q, tensor_of(qv, "bf16"), win, W, K.RowStore(pool, K.DSV4_BF16, D, cnt), dev(idx_o),
                             dev(c.sinks), c.sm_scale, R, c.theta, out_dtype=torch.float32)
    out_o = O.attn(seq, tok, c.pos0, b16(qv), "bf16", f64rows(kv_rot_o, first_tok=[0] * B), W, f64rows(pool_o),
                   "csa", idx=idx_o, sinks=c.sinks, sm_scale=c.sm_scale, rope_dim=R, theta=c.theta)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), out_o, "bf16", "csa layer")
