"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check uses a closed form, a
worked example from the pages, a textbook routine (torch SDPA in fp64, a
sort), brute force, or the independent mask formulation (formulation B).
"""
import json
import os

import numpy as np
import pytest
import torch

import dsv4_synth as S
from oracle import mask_oracle as MB

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def rows(x, kind="f32", **kw):
    return S.rowset_from_values(np.asarray(x, np.float32)[None] if np.ndim(x) == 2 else x, kind, **kw)


def f32(x):
    return np.asarray(x, np.float32)


# --------------------------------------------------------------------------- worked example
def test_worked_example_visibility_and_selection(orc):
    """HF page, 'Attention mask layout': 16 tokens, window 8, m=4, m'=8, top-k 2."""
    g = json.load(open(os.path.join(GOLD, "worked_example_mask.json")))
    Sx, W, m, mh, k = g["S"], g["sliding_window"], g["csa_m"], g["hca_m"], g["index_topk"]
    t = np.arange(Sx)
    assert list(orc.n_visible(t, m, Sx // m)) == g["csa_available"]
    assert list(orc.n_visible(t, mh, Sx // mh)) == g["hca_visible"]
    # selection through the oracle's indexer + top-k on random keys/queries
    rng = np.random.default_rng(0)
    kpool = rows(rng.standard_normal((Sx // m, 8)))
    sc = orc.index_scores(np.zeros(Sx, np.int32), t, f32(rng.standard_normal((Sx, 2, 8))), "f32",
                          rng.standard_normal((Sx, 2)), kpool, m, 1.0)
    idx = orc.topk(sc, orc.n_visible(t, m, Sx // m), k)
    assert list((idx >= 0).sum(1)) == g["csa_selected"]
    for r in range(Sx):     # valid picks first, then the -1 sentinel
        v = idx[r]
        nv = int((v >= 0).sum())
        assert np.all(v[nv:] == -1) and np.all(v[:nv] < g["csa_available"][r])


def test_worked_example_window_and_hca_membership(orc):
    """q = 0 gives o = mean of the visible rows; one-hot rows reveal which rows
    each query sees: the sliding band (cut from row `window` on) and HCA entries."""
    g = json.load(open(os.path.join(GOLD, "worked_example_mask.json")))
    Sx, W, mh = g["S"], g["sliding_window"], g["hca_m"]
    eye = np.eye(Sx, dtype=np.float32)
    win = rows(eye, count=[Sx], first_tok=[0])
    q = np.zeros((Sx, 1, Sx), np.float32)
    o = orc.attn(np.zeros(Sx), np.arange(Sx), [0], q, "f32", win, W, None, "hca", m=mh)
    seen = o[:, 0, :] > 0
    assert list(seen.sum(1)) == g["sliding_row_lengths"]
    for t in range(Sx):
        assert np.allclose(o[t, 0, seen[t]], 1.0 / seen[t].sum(), atol=1e-15)
        assert seen[t, t] and (t < g["sliding_first_cut_row"] or not seen[t, t - W])
    pool = rows(np.eye(Sx // mh, Sx, dtype=np.float32))
    o = orc.attn(np.zeros(Sx), np.arange(Sx), [0], q, "f32", None, 0, pool, "hca", m=mh)
    vis = (o[:, 0, :Sx // mh] > 0).sum(1)
    assert list(vis) == g["hca_visible"]
    first = [int(np.argmax(o[:, 0, w] > 0)) for w in range(Sx // mh)]
    assert first == g["hca_entry_first_visible_t"]


# --------------------------------------------------------------------------- codecs
def test_e4m3_all_codes_match_torch(orc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([orc.e4m3_to_f64(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.nanmax(got) == 448.0


def test_f16_all_codes_match_numpy(orc):
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(c)) for c in codes[::7]])
    r = ref[::7]
    nan = np.isnan(r)
    assert np.array_equal(nan, np.isnan(got)) and np.array_equal(r[~nan], got[~nan])


def test_e2m1_and_e8m0_tables(orc):
    # OCP MX spec: E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; bit 3 is the sign
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = orc.e2m1_to_f64(c)
        assert abs(v) == mags[c & 7] and (np.signbit(v) == bool(c & 8) or v == 0)
    for e in range(255):
        assert orc.e8m0_to_f64(e) == 2.0 ** (e - 127)
    assert np.isnan(orc.e8m0_to_f64(255))


def test_row_formats_decode(orc):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 5, 512)).astype(np.float32)
    rs = S.rowset_from_values(x, "fp8r", tail=64)
    dec = orc.decode(rs)
    # rope channels are bf16-exact; the rest within e4m3 precision (2^-4 relative) of x
    assert np.array_equal(dec[..., 448:], S.bf16_to_f32(S.bf16_bits(x[..., 448:])))
    amax = np.abs(x[..., :448]).max(-1, keepdims=True)
    assert np.all(np.abs(dec[..., :448] - x[..., :448]) <= 2.0 ** -4 * np.abs(x[..., :448]) + amax / 448 * 2.0 ** -9)
    # per-row amax maps to 448 exactly
    assert np.allclose(np.abs(dec[..., :448]).max(-1), amax[..., 0], rtol=1e-7)
    # MXFP4: an exactly representable block decodes exactly
    blk = np.array([0, .5, 1, 1.5, 2, 3, 4, 6] * 4, np.float32) * 0.25
    pk, sc = S.mxfp4_pack(blk[None, None, :])
    assert sc[0, 0, 0] == 127 - 2 + 0  # amax 1.5 -> floor(log2 1.5) - 2 = -2
    dm = orc.decode(S.RowSet("mxfp4", pk, 32, np.array([1], np.int32), blk_scale=sc))
    assert np.array_equal(dm[0, 0], blk)


# --------------------------------------------------------------------------- RoPE
def test_rope_closed_forms(orc):
    D, R = 32, 16
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, D))
    pos = np.array([0, 1, 5, 77, 4096, 2 ** 20, 12345])
    y = orc.rope(x, pos, R, 10000.0, +1)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.array_equal(y[:, :D - R], x[:, :D - R])
    assert np.allclose(orc.rope(y, pos, R, 10000.0, -1), x, atol=1e-12)
    assert np.array_equal(orc.rope(x, pos, 0, 10000.0, +1), x)
    # pair 0 turns at frequency 1: position pi flips it, pi/2 maps (1,0) -> (0,1)
    e = np.zeros((1, D)); e[0, D - R] = 1.0
    assert np.allclose(orc.rope(e, [np.pi], R, 10000.0, +1)[0, D - R:D - R + 2], [-1, 0], atol=1e-15)
    assert np.allclose(orc.rope(e, [np.pi / 2], R, 10000.0, +1)[0, D - R:D - R + 2], [0, 1], atol=1e-15)
    # the last pair turns at theta^(-(R-2)/R): one full turn returns the vector
    e2 = np.zeros((1, D)); e2[0, D - 2] = 1.0
    full = 2 * np.pi / 10000.0 ** (-(R - 2) / R)
    assert np.allclose(orc.rope(e2, [full], R, 10000.0, +1)[0, D - 2:], [1, 0], atol=1e-9)
    # interleaved pairs: a unit vector stays inside its own (2i, 2i+1) pair
    for i in range(R // 2):
        e = np.zeros((1, D)); e[0, D - R + 2 * i] = 1.0
        y = orc.rope(e, [3.3], R, 10000.0, +1)[0]
        nz = set(np.nonzero(np.abs(y) > 1e-15)[0])
        assert nz <= {D - R + 2 * i, D - R + 2 * i + 1}


def test_rope_formulations_agree(orc):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 64))
    pos = rng.integers(0, 2 ** 20, 50)
    a = orc.rope(x, pos, 16, 160000.0, +1)
    b = MB.rope_complex(x, pos, 16, 160000.0, +1)
    assert np.allclose(a, b, rtol=0, atol=1e-11)


# --------------------------------------------------------------------------- compressor
@pytest.mark.parametrize("overlap,m", [(True, 4), (False, 8), (True, 2), (False, 1)])
def test_compressor_convex_and_formulations(orc, overlap, m):
    rng = np.random.default_rng(4 + m)
    Sx, dim = 37, 12
    width = 2 * m if overlap else m
    c = rng.standard_normal((1, Sx, dim)).astype(np.float32)
    z = (3 * rng.standard_normal((1, Sx, dim))).astype(np.float32)
    bias = rng.standard_normal((width, dim))
    a = orc.compress(c, z, bias, m, overlap)[0]
    b = MB.compress_masked(c[0], z[0], bias, m, overlap)
    assert a.shape == (Sx // m, dim)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
    for s in range(Sx // m):   # convexity over each entry's window
        lo = max(0, (s - 1) * m if overlap else s * m)
        hi = (s + 1) * m
        seg = c[0, lo:hi].astype(np.float64)
        assert np.all(a[s] >= seg.min(0) - 1e-12) and np.all(a[s] <= seg.max(0) + 1e-12)


def test_compressor_special_cases(orc):
    rng = np.random.default_rng(5)
    Sx, dim, m = 40, 6, 4
    bias = rng.standard_normal((2 * m, dim))
    z = rng.standard_normal((1, Sx, dim)).astype(np.float32)
    # constant window -> that constant, whatever the gates
    c = np.full((1, Sx, dim), 1.75, np.float32)
    assert np.allclose(orc.compress(c, z, bias, m, True), 1.75, rtol=0, atol=1e-14)
    # uniform gates (z const, bias 0) -> arithmetic mean of the window
    c = rng.standard_normal((1, Sx, dim)).astype(np.float32)
    zc = np.full((1, Sx, dim), 0.3, np.float32)
    a = orc.compress(c, zc, np.zeros((2 * m, dim)), m, True)[0]
    for s in range(Sx // m):
        lo = max(0, (s - 1) * m)
        assert np.allclose(a[s], c[0, lo:(s + 1) * m].astype(np.float64).mean(0), rtol=0, atol=1e-12)
    # a one-hot position bias selects one token of the window: offset j of
    # entry s is token (s-1)m + j (CSA, window [(s-1)m, (s+1)m))
    for j in range(2 * m):
        bj = np.zeros((2 * m, dim)); bj[j] = 60.0
        a = orc.compress(c, np.zeros_like(c), bj, m, True)[0]
        for s in range(Sx // m):
            t = (s - 1) * m + j
            if t >= 0:
                assert np.allclose(a[s], c[0, t], atol=1e-20 + 1e-12)
            else:   # the missing half of entry 0 takes no part: mean of tokens 0..m-1
                assert np.allclose(a[s], c[0, :m].astype(np.float64).mean(0), atol=1e-12)
    # HCA one-hot on offset j -> token s*m + j
    bh = np.zeros((m, dim)); bh[2] = 60.0
    a = orc.compress(c, np.zeros_like(c), bh, m, False)[0]
    assert np.allclose(a, c[0, 2::m][:Sx // m], atol=1e-12)
    # m = 1 without overlap: every entry is its token (identity up to RoPE)
    a = orc.compress(c, z, np.zeros((1, dim)), 1, False)[0]
    assert np.array_equal(a, c[0].astype(np.float64))
    a = orc.compress(c, z, np.zeros((1, dim)), 1, False, rope_dim=4, theta=100.0)[0]
    assert np.allclose(a, orc.rope(c[0], np.arange(Sx), 4, 100.0, +1), atol=1e-14)


def test_compressor_rope_position(orc):
    """Entry s is rotated at pos0 + s*m: with a constant window the pooled value is
    known, so the rotation angle can be read off."""
    Sx, dim, m, R = 32, 8, 4, 4
    c = np.zeros((1, Sx, dim), np.float32); c[..., dim - R] = 1.0
    a = orc.compress(c, np.zeros_like(c), np.zeros((2 * m, dim)), m, True, rope_dim=R, theta=1e4, pos0=[7])[0]
    ang = np.arctan2(a[:, dim - R + 1], a[:, dim - R])
    expect = np.angle(np.exp(1j * (7 + np.arange(Sx // m) * m)))
    assert np.allclose(ang, expect, atol=1e-12)


# --------------------------------------------------------------------------- indexer + top-k
def test_indexer_closed_forms(orc):
    rng = np.random.default_rng(6)
    Sx, m, Di, N = 24, 4, 16, 6
    kp = rng.standard_normal((1, N, Di)).astype(np.float32)
    qi = rng.standard_normal((Sx, 1, Di)).astype(np.float32)
    t = np.arange(Sx)
    sc = orc.index_scores(np.zeros(Sx), t, qi, "f32", np.ones((Sx, 1)), rows(kp[0]), m, 0.5)
    dots = qi[:, 0].astype(np.float64) @ kp[0].T.astype(np.float64)
    vis = np.arange(N)[None] < ((t[:, None] + 1) // m)
    assert np.allclose(np.where(vis, sc, 0), np.where(vis, 0.5 * np.maximum(dots, 0), 0), rtol=1e-13, atol=1e-13)
    assert np.all(np.isneginf(sc[~vis]))
    # heads with all-positive dots are linear: sum_h w_h q_h . k = (sum_h w_h q_h) . k
    H = 3
    qp = np.abs(rng.standard_normal((Sx, H, Di))).astype(np.float32)
    kpp = np.abs(rng.standard_normal((N, Di))).astype(np.float32)
    w = rng.standard_normal((Sx, H))
    sc = orc.index_scores(np.zeros(Sx), t, qp, "f32", w, rows(kpp), m, 1.0)
    lin = np.einsum("th,thd->td", w, qp.astype(np.float64)) @ kpp.T.astype(np.float64)
    assert np.allclose(sc[vis], lin[vis], rtol=1e-12, atol=1e-12)
    # a head whose dot is negative contributes nothing, whatever its weight
    qn = qp.copy(); qn[:, 1] = -qn[:, 1]
    wn = w.copy(); wn[:, 1] = 1e6
    sc2 = orc.index_scores(np.zeros(Sx), t, qn, "f32", wn, rows(kpp), m, 1.0)
    lin2 = np.einsum("th,thd->td", w[:, [0, 2]], qp[:, [0, 2]].astype(np.float64)) @ kpp.T.astype(np.float64)
    assert np.allclose(sc2[vis], lin2[vis], rtol=1e-12, atol=1e-12)


def test_indexer_formulations_agree(orc):
    rng = np.random.default_rng(7)
    Sx, m, H, Di = 40, 4, 4, 32
    kp = rng.standard_normal((Sx // m, Di)).astype(np.float32)
    qi = rng.standard_normal((Sx, H, Di)).astype(np.float32)
    w = rng.standard_normal((Sx, H))
    a = orc.index_scores(np.zeros(Sx), np.arange(Sx), qi, "f32", w, rows(kp), m, 0.3)
    b = MB.index_scores_dense(qi, w, kp, m, 0.3)
    fin = np.isfinite(b)
    assert np.array_equal(fin, np.isfinite(a))
    assert np.allclose(a[fin], b[fin], rtol=1e-12, atol=1e-12)


def test_topk_brute_force_and_ties(orc):
    rng = np.random.default_rng(8)
    n_q, nmax, k = 60, 50, 7
    sc = np.round(rng.standard_normal((n_q, nmax)), 1)      # many exact ties
    nv = rng.integers(0, nmax + 1, n_q)
    masked = np.where(np.arange(nmax)[None] < nv[:, None], sc, -np.inf)
    got = orc.topk(masked, nv, k)
    ref = MB.topk_by_sort(masked, k)
    assert np.array_equal(got, ref)
    assert np.array_equal((got >= 0).sum(1), np.minimum(k, nv))
    # k >= n: every visible entry; all-equal scores: the first k indices
    got = orc.topk(np.zeros((3, 10)), [10, 4, 0], 6)
    assert got.tolist() == [[0, 1, 2, 3, 4, 5], [0, 1, 2, 3, -1, -1], [-1] * 6]


def test_topk_invariant_to_positive_weight_scale(orc):
    rng = np.random.default_rng(9)
    Sx, m, H, Di = 64, 4, 4, 32
    kp = rows(rng.standard_normal((Sx // m, Di)))
    qi = rng.standard_normal((Sx, H, Di)).astype(np.float32)
    w = rng.standard_normal((Sx, H))
    t = np.arange(Sx)
    nv = orc.n_visible(t, m, Sx // m)
    a = orc.topk(orc.index_scores(np.zeros(Sx), t, qi, "f32", w, kp, m, 1.0), nv, 5)
    b = orc.topk(orc.index_scores(np.zeros(Sx), t, qi, "f32", 8.0 * w, kp, m, 1.0), nv, 5)
    assert np.array_equal(a, b)
    # all dots negative -> all scores 0 -> first k visible entries
    kn = rows(-np.abs(rng.standard_normal((Sx // m, Di))))
    qn = np.abs(qi)
    c = orc.topk(orc.index_scores(np.zeros(Sx), t, qn, "f32", w, kn, m, 1.0), nv, 5)
    for r in range(Sx):
        n = min(5, nv[r])
        assert c[r].tolist() == list(range(n)) + [-1] * (5 - n)


# --------------------------------------------------------------------------- attention
def _sdpa_with_sink(q, K, V, sinks, allowed, scale):
    """Textbook pin: torch SDPA in fp64 on the CPU over [0 ; K] / [0 ; V] with the
    sink as the logit of the zero key (column 0 of a float mask)."""
    Sx, H, D = q.shape
    Kz = torch.cat([torch.zeros(1, D, dtype=torch.float64), torch.from_numpy(K)], 0)
    Vz = torch.cat([torch.zeros(1, D, dtype=torch.float64), torch.from_numpy(V)], 0)
    mask = torch.where(torch.from_numpy(allowed), 0.0, float("-inf")).to(torch.float64)
    col0 = torch.tensor(sinks, dtype=torch.float64)[:, None, None].expand(H, Sx, 1) if sinks is not None \
        else torch.full((H, Sx, 1), float("-inf"), dtype=torch.float64)
    full = torch.cat([col0, mask[None].expand(H, -1, -1)], -1)[None]
    qq = torch.from_numpy(q).permute(1, 0, 2)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qq, Kz[None, None].expand(1, H, -1, -1),
                                                         Vz[None, None].expand(1, H, -1, -1),
                                                         attn_mask=full, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_hca_m1_no_window_is_causal_mqa_with_sink(orc):
    rng = np.random.default_rng(10)
    Sx, H, D = 33, 4, 16
    q = rng.standard_normal((Sx, H, D)).astype(np.float32)
    c = rng.standard_normal((1, Sx, D)).astype(np.float32)
    z = rng.standard_normal((1, Sx, D)).astype(np.float32)
    sinks = rng.standard_normal(H)
    pool = orc.compress(c, z, rng.standard_normal((1, D)), 1, False)      # m' = 1: the tokens
    o = orc.attn(np.zeros(Sx), np.arange(Sx), [0], q, "f32", None, 0,
                 rows(pool[0].astype(np.float32)), "hca", m=1, sinks=sinks, sm_scale=0.25)
    causal = np.tril(np.ones((Sx, Sx), bool))
    ref = _sdpa_with_sink(q.astype(np.float64), pool[0], pool[0], sinks, causal, 0.25)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)


def test_window_only_and_sink_limits(orc):
    rng = np.random.default_rng(11)
    Sx, H, D, W = 30, 3, 8, 5
    q = rng.standard_normal((Sx, H, D)).astype(np.float32)
    kv = rng.standard_normal((Sx, D)).astype(np.float32)
    sinks = rng.standard_normal(H)
    win = rows(kv, count=[Sx], first_tok=[0])
    band = (np.arange(Sx)[None] <= np.arange(Sx)[:, None]) & (np.arange(Sx)[None] > np.arange(Sx)[:, None] - W)
    pool = rows(rng.standard_normal((Sx // 4, D)))
    empty_idx = np.full((Sx, 3), -1, np.int32)
    o = orc.attn(np.zeros(Sx), np.arange(Sx), [0], q, "f32", win, W, pool, "csa", idx=empty_idx,
                 sinks=sinks, sm_scale=0.5)
    ref = _sdpa_with_sink(q.astype(np.float64), kv.astype(np.float64), kv.astype(np.float64), sinks, band, 0.5)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    o = orc.attn(np.zeros(Sx), np.arange(Sx), [0], q, "f32", win, W, None, "hca", m=4, sinks=None, sm_scale=0.5)
    ref = _sdpa_with_sink(q.astype(np.float64), kv.astype(np.float64), kv.astype(np.float64), None, band, 0.5)
    assert np.allclose(o, ref, rtol=1e-12, atol=1e-13)
    big = orc.attn(np.zeros(Sx), np.arange(Sx), [0], q, "f32", win, W, None, "hca", m=4,
                   sinks=np.full(H, 400.0), sm_scale=0.5)
    assert np.max(np.abs(big)) < 1e-150


def test_zero_query_closed_form(orc):
    rng = np.random.default_rng(12)
    Sx, H, D, W, m = 21, 2, 8, 4, 4
    kv = rng.standard_normal((Sx, D)).astype(np.float32)
    pool = rng.standard_normal((Sx // m, D)).astype(np.float32)
    sinks = rng.standard_normal(H)
    o = orc.attn(np.zeros(Sx), np.arange(Sx), [0], np.zeros((Sx, H, D), np.float32), "f32",
                 rows(kv, count=[Sx], first_tok=[0]), W, rows(pool), "hca", m=m, sinks=sinks)
    for t in range(Sx):
        X = list(kv[max(0, t - W + 1):t + 1]) + list(pool[:(t + 1) // m])
        X = np.array(X, np.float64)
        for h in range(H):
            assert np.allclose(o[t, h], X.sum(0) / (len(X) + np.exp(sinks[h])), rtol=1e-13, atol=1e-14)


def _tiny_layer(orc, seed=13, Sx=48, H=4, D=16, R=8, W=6, m=4, k=3, pos0=0, theta=1000.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Sx, H, D)).astype(np.float32)
    kv = rng.standard_normal((Sx, D)).astype(np.float32)
    c = rng.standard_normal((1, Sx, D)).astype(np.float32)
    z = rng.standard_normal((1, Sx, D)).astype(np.float32)
    bias = 0.1 * rng.standard_normal((2 * m, D))
    sinks = rng.standard_normal(H)
    pool = orc.compress(c, z, bias, m, True, rope_dim=R, theta=theta, pos0=[pos0])[0]
    kv_rot = orc.rope(kv, pos0 + np.arange(Sx), R, theta, +1)
    N = Sx // m
    sc = rng.standard_normal((Sx, N))
    nv = orc.n_visible(np.arange(Sx), m, N)
    idx = orc.topk(np.where(np.arange(N)[None] < nv[:, None], sc, -np.inf), nv, k)
    return dict(q=q, kv_rot=kv_rot, pool=pool, idx=idx, sinks=sinks, Sx=Sx, H=H, D=D, R=R, W=W, m=m,
                theta=theta, pos0=pos0)


def _f64rows(x, first_tok=None):
    x = np.asarray(x, np.float64)
    n = x.shape[0]
    return S.RowSet("f64", x[None].copy().view(np.uint8).reshape(1, n, -1), x.shape[1],
                    np.array([n], np.int32),
                    first_tok=None if first_tok is None else np.array([first_tok], np.int32))


def _csa(orc, L, idx=None, q=None):
    Sx = L["Sx"]
    return orc.attn(np.zeros(Sx), np.arange(Sx), [L["pos0"]], L["q"] if q is None else q, "f32",
                    _f64rows(L["kv_rot"], first_tok=0), L["W"], _f64rows(L["pool"]),
                    "csa", idx=L["idx"] if idx is None else idx, sinks=L["sinks"],
                    sm_scale=1 / np.sqrt(L["D"]), rope_dim=L["R"], theta=L["theta"])


def _hca(orc, L, m=None):
    Sx = L["Sx"]
    return orc.attn(np.zeros(Sx), np.arange(Sx), [L["pos0"]], L["q"], "f32",
                    _f64rows(L["kv_rot"], first_tok=0), L["W"], _f64rows(L["pool"]),
                    "hca", m=L["m"] if m is None else m, sinks=L["sinks"],
                    sm_scale=1 / np.sqrt(L["D"]), rope_dim=L["R"], theta=L["theta"])


def test_attention_formulations_agree(orc):
    L = _tiny_layer(orc)
    a = _csa(orc, L)
    b = MB.csa_attention(L["q"], L["kv_rot"], L["pool"], L["idx"], L["sinks"], L["W"],
                         1 / np.sqrt(L["D"]), L["R"], L["theta"], L["pos0"])
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)
    a = _hca(orc, L)
    b = MB.hca_attention(L["q"], L["kv_rot"], L["pool"], L["m"], L["sinks"], L["W"],
                         1 / np.sqrt(L["D"]), L["R"], L["theta"], L["pos0"])
    assert np.allclose(a, b, rtol=1e-12, atol=1e-13)


def test_topk_full_pool_reproduces_dense(orc):
    """Selecting every visible entry (top-k = N) is HCA-style dense attention
    over the same pool with the same visibility stride."""
    L = _tiny_layer(orc, k=12)
    N = L["pool"].shape[0]
    nv = orc.n_visible(np.arange(L["Sx"]), L["m"], N)
    idx_all = orc.topk(np.where(np.arange(N)[None] < nv[:, None], 0.0, -np.inf), nv, N)
    assert np.allclose(_csa(orc, L, idx=idx_all), _hca(orc, L), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("delta", [1, 3, 4096, 2 ** 20 - 48])
def test_relative_position_invariance(orc, delta):
    """Shifting every position by delta leaves the output unchanged: keys and the
    query turn together and the output slice is turned back (HF page, partial
    RoPE bullet).  The pool is rebuilt at the shifted positions."""
    L0 = _tiny_layer(orc, pos0=0)
    L1 = _tiny_layer(orc, pos0=delta)
    L1["idx"] = L0["idx"]
    assert np.allclose(_csa(orc, L0), _csa(orc, L1), rtol=1e-9, atol=1e-10)
    assert np.allclose(_hca(orc, L0), _hca(orc, L1), rtol=1e-9, atol=1e-10)


def test_decode_step_equals_last_prefill_row(orc):
    """O8: a decode query at t = L-1 with a window cache holding tokens L-W..L-1
    (first_tok = L-W) is the last row of the prefill computation."""
    L = _tiny_layer(orc, Sx=45, W=6, k=4)
    Sx, W = L["Sx"], L["W"]
    full = _hca(orc, L)
    winc = _f64rows(L["kv_rot"][Sx - W:], first_tok=Sx - W)
    o = orc.attn([0], [Sx - 1], [L["pos0"]], L["q"][Sx - 1:], "f32", winc, W, _f64rows(L["pool"]), "hca",
                 m=L["m"], sinks=L["sinks"], sm_scale=1 / np.sqrt(L["D"]), rope_dim=L["R"], theta=L["theta"])
    assert np.allclose(o[0], full[-1], rtol=1e-13, atol=1e-14)


def test_indexer_reads_mxfp4_as_decoded_values(orc):
    rng = np.random.default_rng(14)
    N, H, Di, m = 30, 4, 64, 4
    keys = S.rowset_from_values(rng.standard_normal((1, N, Di)), "mxfp4")
    qpk, qsc = S.mxfp4_pack(rng.standard_normal((2, H, Di)).astype(np.float32))
    w = rng.standard_normal((2, H))
    tok = [N * m - 1, 57]
    a = orc.index_scores([0, 0], tok, qpk, "mxfp4", w, keys, m, 0.7, q_scale=qsc)
    qdec = orc.decode(S.RowSet("mxfp4", qpk.reshape(1, 2 * H, -1), Di, np.array([2 * H], np.int32),
                               blk_scale=qsc.reshape(1, 2 * H, -1)))[0].reshape(2, H, Di)
    kdec = orc.decode(keys)[0]
    # same scores from the decoded values handed over in fp64 (the codec itself
    # is pinned by the table tests above; the arithmetic by the closed forms)
    ref = orc.index_scores([0, 0], tok, qdec, "f64", w, _f64rows(kdec), m, 0.7)
    for r, t in enumerate(tok):
        n = min(N, (t + 1) // m)
        assert np.array_equal(a[r, :n], ref[r, :n])
        assert np.all(np.isneginf(a[r, n:]))
