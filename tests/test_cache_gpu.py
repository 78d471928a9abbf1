"""Streaming cache maintenance (dsv4_cache_append) and ring windows.

* After every append of a schedule that mixes a prefill-sized append, ragged
  multi-token appends (some sequences taking none) and single-token decode
  steps, the cache must hold exactly what the batch calls produce from each
  sequence's whole history: pool rows = dsv4_compress (+ dsv4_quantize), window
  ring rows = dsv4_rope (+ dsv4_quantize) of the newest tokens, bit for bit,
  and len / count / window count / first token must follow the token counts.
* Against the oracle: the streamed pools and window rows decode to the
  oracle's pooled / rotated values within the storage format's rounding.
* A decode step over the streamed cache (indexer + top-k on the streamed
  indexer pool, attention over the ring window and the streamed pool) against
  the oracle computing on caches it builds itself.
* Attention over a ring window equals attention over the same rows stored
  linearly, bit for bit, on every attention path.
"""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import assert_close, check_topk, dev, tensor_of, upload_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


F32, BF16, FP8R, MXFP4, F16 = 0, 1, 2, 3, 4
CASES = {
    # CSA: overlapping windows of 2m, FP8 K=V rows with bf16 rope channels, MXFP4 indexer keys
    "csa_fp8_mxfp4": dict(m=4, overlap=True, D=512, R=64, kv_dtype=FP8R, tail=64, win_dtype=FP8R, W=128,
                          idx_dim=128, idx_dtype=MXFP4, xkind="bf16"),
    "csa_bf16": dict(m=4, overlap=True, D=512, R=64, kv_dtype=BF16, tail=0, win_dtype=BF16, W=64,
                     idx_dim=128, idx_dtype=BF16, xkind="f32"),
    # HCA: non-overlapping windows, one stream
    "hca_fp8": dict(m=16, overlap=False, D=512, R=64, kv_dtype=FP8R, tail=64, win_dtype=FP8R, W=32,
                    idx_dim=0, idx_dtype=0, xkind="bf16"),
    "hca128_f16": dict(m=128, overlap=False, D=256, R=32, kv_dtype=F16, tail=0, win_dtype=F16, W=16,
                       idx_dim=0, idx_dtype=0, xkind="f32"),
    # the small fp32 shapes (dim 64, stride 2) with fp32 pools, window and indexer keys
    "csa_f32_small": dict(m=2, overlap=True, D=64, R=16, kv_dtype=F32, tail=0, win_dtype=F32, W=24,
                          idx_dim=64, idx_dtype=F32, xkind="f32"),
}
B = 3
POS0 = np.array([0, 1000, 77], np.int64)
THETA = 1.6e5
# (n, n_new per sequence or None = n for all)
SCHEDULE = [(37, [37, 20, 0]), (1, None), (1, None), (1, None), (9, [9, 3, 5]), (1, [1, 0, 1]), (1, None),
            (200, [200, 131, 180]), (1, None), (1, None), (300, [300, 0, 257]), (1, None)]


class Stream:
    """Runs the schedule on the GPU and keeps each sequence's host history."""

    def __init__(self, K, cfg, seed):
        self.cfg, self.rng = cfg, np.random.default_rng(seed)
        c = cfg
        span = 2 * c["m"] if c["overlap"] else c["m"]
        total = sum(n for n, _ in SCHEDULE)
        self.cap = total // c["m"] + 2
        self.kv_bias = (0.1 * self.rng.standard_normal((span, c["D"]))).astype(np.float32)
        self.idx_bias = ((0.1 * self.rng.standard_normal((span, c["idx_dim"]))).astype(np.float32)
                         if c["idx_dim"] else None)
        self.cache = K.DecodeCache(B, c["m"], c["overlap"], c["D"], dev(self.kv_bias), self.cap, c["W"],
                                   rope_dim=c["R"], rope_theta=THETA, kv_dtype=c["kv_dtype"], kv_tail=c["tail"],
                                   win_dtype=c["win_dtype"], idx_dim=c["idx_dim"],
                                   idx_bias=dev(self.idx_bias) if c["idx_dim"] else None,
                                   idx_dtype=c["idx_dtype"] if c["idx_dim"] else MXFP4, pos0=dev(POS0))
        self.hist = {k: [np.zeros((0, d), np.float32) for _ in range(B)]
                     for k, d in (("kv", c["D"]), ("c", c["D"]), ("z", c["D"]),
                                  ("ci", c["idx_dim"]), ("zi", c["idx_dim"]))}

    def draw(self, n, dim):
        x = self.rng.standard_normal((B, n, dim)).astype(np.float32)
        return S.bf16_to_f32(S.bf16_bits(x)) if self.cfg["xkind"] == "bf16" else x

    def append(self, n, n_new):
        c = self.cfg
        ins = {"kv": self.draw(n, c["D"]), "c": self.draw(n, c["D"]), "z": self.draw(n, c["D"])}
        if c["idx_dim"]:
            ins["ci"] = self.draw(n, c["idx_dim"])
            ins["zi"] = self.draw(n, c["idx_dim"])
        nn = [n] * B if n_new is None else n_new
        for k, v in ins.items():
            for b in range(B):
                self.hist[k][b] = np.concatenate([self.hist[k][b], v[b, :nn[b]]])
        t = {k: tensor_of(v, c["xkind"]) for k, v in ins.items()}
        self.cache.append(t["kv"], t["c"], t["z"], t.get("ci"), t.get("zi"),
                          n_new=None if n_new is None else dev(np.asarray(n_new, np.int32)))

    def lengths(self):
        return np.array([len(h) for h in self.hist["kv"]], np.int64)


def _stored(K, x: torch.Tensor, dtype: int, tail: int):
    """Rows x [n, dim] fp32 in storage form via the batch calls: (bytes, row_scale, blk_scale)."""
    if dtype == FP8R:
        r, s = K.dsv4_quantize(x, FP8R, tail)
        return r, s, None
    if dtype == MXFP4:
        r, s = K.dsv4_quantize(x, MXFP4)
        return r, None, s
    t = {F32: torch.float32, BF16: torch.bfloat16, F16: torch.float16}[dtype]
    return x.to(t).contiguous().view(torch.uint8).reshape(x.shape[0], -1), None, None


def _check_against_batch(K, st: Stream, what: str):
    c, cache = st.cfg, st.cache
    L = st.lengths()
    torch.cuda.synchronize()
    assert np.array_equal(cache.len.cpu().numpy(), L), f"{what}: len"
    assert np.array_equal(cache.kv["count"].cpu().numpy(), np.minimum(L // c["m"], st.cap)), f"{what}: count"
    wc = np.minimum(L, c["W"])
    assert np.array_equal(cache.win_count.cpu().numpy(), wc), f"{what}: window count"
    assert np.array_equal(cache.win_first.cpu().numpy(), L - wc), f"{what}: window first token"
    streams = [("kv", "c", "z", c["D"], c["R"], c["kv_dtype"], c["tail"], st.kv_bias, cache.kv)]
    if c["idx_dim"]:
        streams.append(("idx", "ci", "zi", c["idx_dim"], 0, c["idx_dtype"], 0, st.idx_bias, cache.idx))
    for b in range(B):
        Lb = int(L[b])
        N = Lb // c["m"]
        for name, kc, kz, dim, R, dt, tail, bias, sd in streams:
            if N == 0:
                continue
            hc = tensor_of(st.hist[kc][b][None], c["xkind"])
            hz = tensor_of(st.hist[kz][b][None], c["xkind"])
            ref = K.dsv4_compress(hc, hz, dev(bias), c["m"], c["overlap"], R, THETA, pos0=dev(POS0[b:b + 1]),
                                  out_dtype=torch.float32)[0]
            rows, rsc, bsc = _stored(K, ref, dt, tail)
            got = sd["pool"][b, :N]
            assert torch.equal(got, rows), f"{what}: {name} pool rows of sequence {b}"
            if rsc is not None:
                assert torch.equal(sd["row_scale"][b, :N], rsc), f"{what}: {name} row scales of sequence {b}"
            if bsc is not None:
                assert torch.equal(sd["blk_scale"][b, :N], bsc), f"{what}: {name} block scales of sequence {b}"
        if Lb == 0:
            continue
        j = np.arange(Lb - wc[b], Lb)
        kvr = K.dsv4_rope(tensor_of(st.hist["kv"][b][j], c["xkind"]), dev(POS0[b] + j), c["R"], THETA,
                          out_dtype=torch.float32)
        rows, rsc, _ = _stored(K, kvr, c["win_dtype"], c["tail"] if c["win_dtype"] == FP8R else 0)
        slots = torch.from_numpy(j % c["W"]).cuda()
        assert torch.equal(cache.win[b].index_select(0, slots), rows), f"{what}: window rows of sequence {b}"
        if rsc is not None:
            assert torch.equal(cache.win_scale[b].index_select(0, slots), rsc), f"{what}: window scales {b}"


@pytest.mark.parametrize("name", list(CASES))
def test_stream_equals_batch(K, name):
    """Every append leaves the cache equal, bit for bit, to the batch compressor
    / rope / quantiser over each sequence's whole history."""
    st = Stream(K, CASES[name], seed=len(name) * 17)
    for i, (n, nn) in enumerate(SCHEDULE):
        say(name, "append", i, n, nn)
        st.append(n, nn)
        _check_against_batch(K, st, f"{name} after append {i}")


def _kind(dtype):
    return {F32: "f32", BF16: "bf16", F16: "f16", FP8R: "fp8r", MXFP4: "mxfp4"}[dtype]


def _gpu_rowset(t_rows, dtype, dim, tail=0, rsc=None, bsc=None):
    return S.RowSet(_kind(dtype), t_rows.cpu().numpy(), dim, np.full(t_rows.shape[0], t_rows.shape[1], np.int32),
                    tail=tail, row_scale=None if rsc is None else rsc.cpu().numpy(),
                    blk_scale=None if bsc is None else bsc.cpu().numpy())


def _within_format(dec, ref, dtype, tail, what):
    """|stored - exact| within the rounding of the format (half a step of the
    code grid at the value, from the oracle's own row / block maxima), plus
    fp32 slack for the GPU's fp32 pooling."""
    ref = np.asarray(ref, np.float64)
    slack = 1e-5 * np.abs(ref) + 1e-6
    if dtype == F32:
        bound = slack
    elif dtype in (BF16, F16):
        bound = (2.0 ** -8 if dtype == BF16 else 2.0 ** -11) * np.abs(ref) + slack
    elif dtype == FP8R:
        nq = ref.shape[-1] - tail
        s = np.abs(ref[..., :nq]).max(-1, keepdims=True) / 448.0
        b8 = 2.0 ** -4 * np.abs(ref[..., :nq]) + s * 2.0 ** -10
        bt = 2.0 ** -8 * np.abs(ref[..., nq:])
        bound = np.concatenate([b8, bt], -1) * (1 + 1e-4) + slack
    else:   # MXFP4: 32-channel blocks, scale 2^(floor(log2 amax) - 2), saturating at 6 X
        blk = ref.reshape(*ref.shape[:-1], -1, 32)
        X = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(blk).max(-1, keepdims=True), 1e-300))) - 2)
        b4 = np.maximum(0.25 * np.abs(blk), 0.25 * X) + np.maximum(0.0, np.abs(blk) - 6 * X)
        bound = b4.reshape(ref.shape) * (1 + 1e-4) + slack
    err = np.abs(dec - ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} outside the format's rounding; " \
                          f"worst err {err.max():.3e}"


@pytest.mark.parametrize("name", ["csa_fp8_mxfp4", "hca_fp8", "hca128_f16", "csa_f32_small"])
def test_stream_against_oracle(K, name):
    """The streamed cache decodes to the oracle's pooled and rotated values."""
    c = CASES[name]
    st = Stream(K, c, seed=5 + len(name))
    for n, nn in SCHEDULE:
        st.append(n, nn)
    torch.cuda.synchronize()
    say(name, "lengths", st.lengths().tolist())
    L = st.lengths()
    store = "bf16" if c["xkind"] == "bf16" else "f32"
    enc = (lambda x: S.bf16_bits(x)) if store == "bf16" else (lambda x: x)
    streams = [("c", "z", c["D"], c["R"], c["kv_dtype"], c["tail"], st.kv_bias, st.cache.kv)]
    if c["idx_dim"]:
        streams.append(("ci", "zi", c["idx_dim"], 0, c["idx_dtype"], 0, st.idx_bias, st.cache.idx))
    for b in range(B):
        Lb = int(L[b])
        N = Lb // c["m"]
        for kc, kz, dim, R, dt, tail, bias, sd in streams:
            if N == 0:
                continue
            ref = O.compress(enc(st.hist[kc][b][None]), enc(st.hist[kz][b][None]), bias, c["m"], c["overlap"], R,
                             THETA, POS0[b:b + 1], kind=store)[0]
            rs = _gpu_rowset(sd["pool"][b:b + 1, :N], dt, dim, tail,
                             None if sd["row_scale"] is None else sd["row_scale"][b:b + 1, :N],
                             None if sd["blk_scale"] is None else sd["blk_scale"][b:b + 1, :N])
            _within_format(O.decode(rs)[0], ref, dt, tail, f"{name} pool of sequence {b} (dim {dim})")
        wc = min(Lb, c["W"])
        if wc == 0:
            continue
        j = np.arange(Lb - wc, Lb)
        ref = O.rope(st.hist["kv"][b][j].astype(np.float64), POS0[b] + j, c["R"], THETA, +1)
        wt = c["tail"] if c["win_dtype"] == FP8R else 0
        slots = j % c["W"]
        rs = _gpu_rowset(st.cache.win[b:b + 1, slots], c["win_dtype"], c["D"], wt,
                         None if st.cache.win_scale is None else st.cache.win_scale[b:b + 1, slots])
        _within_format(O.decode(rs)[0], ref, c["win_dtype"], wt, f"{name} window of sequence {b}")


def _oracle_cache(st: Stream):
    """The oracle's own cache after the schedule: pooled by O2, rotated by O1 and
    stored with the oracle's encoders, linear windows."""
    c = st.cfg
    L = st.lengths()
    store = "bf16" if c["xkind"] == "bf16" else "f32"
    enc = (lambda x: S.bf16_bits(x)) if store == "bf16" else (lambda x: x)
    Nmax = int((L // c["m"]).max())
    D, tail, W = c["D"], c["tail"], c["W"]

    def pack(x, dt, tl):
        x = x.astype(np.float32)
        if dt == FP8R:
            r, s = O.quantize_fp8r(x, tl)
            return r, s, None
        if dt == MXFP4:
            r, s = O.quantize_mxfp4(x)
            return r, None, s
        return S.rowset_from_values(x, _kind(dt)).data, None, None

    def pool(kc, kz, dim, R, dt, tl, bias):
        vals = np.zeros((B, Nmax, dim))
        for b in range(B):
            N = int(L[b]) // c["m"]
            if N:
                vals[b, :N] = O.compress(enc(st.hist[kc][b][None]), enc(st.hist[kz][b][None]), bias, c["m"],
                                         c["overlap"], R, THETA, POS0[b:b + 1], kind=store)[0]
        r, s, bs = pack(vals, dt, tl)
        return S.RowSet(_kind(dt), r, dim, (L // c["m"]).astype(np.int32), tail=tl, row_scale=s, blk_scale=bs)

    kvp = pool("c", "z", D, c["R"], c["kv_dtype"], tail, st.kv_bias)
    idp = pool("ci", "zi", c["idx_dim"], 0, c["idx_dtype"], 0, st.idx_bias) if c["idx_dim"] else None
    wvals = np.zeros((B, W, D))
    wc = np.minimum(L, W)
    for b in range(B):
        j = np.arange(L[b] - wc[b], L[b])
        wvals[b, :wc[b]] = O.rope(st.hist["kv"][b][j].astype(np.float64), POS0[b] + j, c["R"], THETA, +1)
    wt = tail if c["win_dtype"] == FP8R else 0
    r, s, _ = pack(wvals, c["win_dtype"], wt)
    win = S.RowSet(_kind(c["win_dtype"]), r, D, wc.astype(np.int32), tail=wt, row_scale=s,
                   first_tok=(L - wc).astype(np.int32))
    return kvp, idp, win


@pytest.mark.parametrize("name", ["csa_fp8_mxfp4", "hca_fp8"])
def test_decode_over_streamed_cache(K, name):
    """One decode step over the cache the appends maintained, against the
    oracle computing on the cache it builds itself from the same tokens."""
    c = CASES[name]
    st = Stream(K, c, seed=99 + len(name))
    for n, nn in SCHEDULE:
        st.append(n, nn)
    # one more decode token for every sequence, then attend from it
    st.append(1, None)
    torch.cuda.synchronize()
    L = st.lengths()
    say(name, "decode at lengths", L.tolist())
    rng = np.random.default_rng(7)
    H, D, R, W, m = 64, c["D"], c["R"], c["W"], c["m"]
    q = S.bf16_to_f32(S.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32)))
    sinks = rng.standard_normal(H).astype(np.float32)
    seq, tok = np.arange(B, dtype=np.int32), (L - 1).astype(np.int32)
    Q = K.QueryRows(dev(seq), dev(tok), dev(POS0), B)
    kvp, idp, win = _oracle_cache(st)
    if name.startswith("csa"):
        k = 64
        Hi, Di = 64, c["idx_dim"]
        w = rng.standard_normal((B, Hi)).astype(np.float32)
        qi_pk, qi_sc = S.mxfp4_pack(rng.standard_normal((B, Hi, Di)).astype(np.float32))
        scale = 1 / np.sqrt(Hi * Di)
        idx_g = K.dsv4_index_topk(Q, dev(qi_pk), dev(w), st.cache.idx_pool(), m, k, scale, q_idx_scale=dev(qi_sc))
        sc_o = O.index_scores(seq, tok, qi_pk, "mxfp4", w, idp, m, scale, q_scale=qi_sc)
        nvis = O.n_visible(tok, m, idp.count)
        torch.cuda.synchronize()
        # keys pooled in fp32 (GPU) and fp64 (oracle) may quantise to
        # neighbouring E2M1 codes: the end-to-end gap bound applies to the
        # streamed pool; over the oracle's stored pool the 1e-5 rule applies
        res = check_topk(idx_g.cpu().numpy(), sc_o, nvis, k, "top-k over the streamed indexer pool", gap=1e-3)
        say("top-k rows exact / near-tie", res)
        idx_s = K.dsv4_index_topk(Q, dev(qi_pk), dev(w), upload_rows(idp), m, k, scale, q_idx_scale=dev(qi_sc))
        torch.cuda.synchronize()
        say("shared-key top-k", check_topk(idx_s.cpu().numpy(), sc_o, nvis, k, "top-k over stored keys"))
        idx_o = O.topk(sc_o, nvis, k)
        out = K.dsv4_sparse_attn(Q, tensor_of(q, "bf16"), st.cache.window(), W, st.cache.kv_pool(), dev(idx_o),
                                 dev(sinks), 1 / np.sqrt(D), R, THETA, out_dtype=torch.float32)
        ref = O.attn(seq, tok, POS0, S.bf16_bits(q), "bf16", win, W, kvp, "csa", idx=idx_o, sinks=sinks,
                     sm_scale=1 / np.sqrt(D), rope_dim=R, theta=THETA)
    else:
        out = K.dsv4_hca_attn(Q, tensor_of(q, "bf16"), st.cache.window(), W, st.cache.kv_pool(), m, dev(sinks),
                              1 / np.sqrt(D), R, THETA, out_dtype=torch.float32)
        ref = O.attn(seq, tok, POS0, S.bf16_bits(q), "bf16", win, W, kvp, "hca", m=m, sinks=sinks,
                     sm_scale=1 / np.sqrt(D), rope_dim=R, theta=THETA)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "bf16", f"{name} decode over the streamed cache")


@pytest.mark.parametrize("kind,qkind,T,W", [("fp8r", "bf16", 5, 128), ("f16", "bf16", 300, 64),
                                            ("bf16", "bf16", 7, 96), ("f32", "f32", 6, 40)])
def test_ring_window_equals_linear(K, kind, qkind, T, W):
    """A window kept as a ring (token j at row j mod W) gives the same bits as
    the same rows stored in token order, and matches the oracle."""
    say("ring window", kind, qkind, T, W)
    rng = np.random.default_rng(3 + T)
    D, R, H = (512, 64, 64) if qkind == "bf16" else (64, 16, 8)
    Bq = 3
    L = np.array([W + 37, 3 * W + 5, W - 9], np.int64)       # wrapped, wrapped twice, not yet full
    vals = rng.standard_normal((Bq, W, D)).astype(np.float32)
    wc = np.minimum(L, W)
    lin = S.rowset_from_values(vals, kind, tail=R if kind == "fp8r" else 0, count=wc, first_tok=L - wc)
    # ring: linear row i (token L - wc + i) goes to slot (L - wc + i) mod W
    ring_data = np.zeros_like(lin.data)
    ring_sc = None if lin.row_scale is None else np.zeros_like(lin.row_scale)
    for b in range(Bq):
        for i in range(wc[b]):
            sl = (L[b] - wc[b] + i) % W
            ring_data[b, sl] = lin.data[b, i]
            if ring_sc is not None:
                ring_sc[b, sl] = lin.row_scale[b, i]
    ring = S.RowSet(kind, ring_data, D, lin.count, tail=lin.tail, row_scale=ring_sc, first_tok=lin.first_tok)
    # queries: T rows spread over the sequences, the newest tokens of each
    seq = np.arange(T, dtype=np.int32) % Bq
    tok = (L[seq] - 1 - (np.arange(T) // Bq) % L[seq]).astype(np.int32)   # newest first, all >= 0
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    if qkind == "bf16":
        q = S.bf16_to_f32(S.bf16_bits(q))
    sinks = rng.standard_normal(H).astype(np.float32)
    Q = K.QueryRows(dev(seq), dev(tok), dev(np.zeros(Bq, np.int64)), Bq)
    rs_lin = upload_rows(lin)
    rs_ring = upload_rows(ring)
    rs_ring.ring = True
    outs = [K.dsv4_sparse_attn(Q, tensor_of(q, qkind), rs, W, None, None, dev(sinks), 1 / np.sqrt(D), R, 1e4,
                               out_dtype=torch.float32) for rs in (rs_lin, rs_ring)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "ring and linear windows differ"
    ref = O.attn(seq, tok, np.zeros(Bq, np.int64), S.bf16_bits(q) if qkind == "bf16" else q, qkind, lin, W,
                 None, "csa", idx=None, sinks=sinks, sm_scale=1 / np.sqrt(D), rope_dim=R,
                 theta=1e4)
    assert_close(outs[1].cpu().numpy(), ref, "bf16" if qkind == "bf16" else "f32", "ring window vs oracle")
