"""Diagnostic counters of the attention calls (dsv4_set_diagnostics).  A pick
entry that is neither the -1 sentinel nor a pool entry below the sequence's
count (HF DeepSeek-V4 page, "Attention mask layout": -1 marks an unused slot)
is counted once per call, whatever the split of its query over workgroups, and
attention treats it exactly like -1: the outputs equal, bit for bit, those of
the same call with such entries set to -1.  Checked on the FP8 decode path
(rows split over several workgroups) and on the fp16 prefill path."""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import dev, tensor_of, upload_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    prev = K.dsv4_set_diagnostics(True)
    K.dsv4_read_diagnostics(reset=True)
    yield K
    K.dsv4_set_diagnostics(prev)
    K.dsv4_read_diagnostics(reset=True)


def plant(idx, counts, rng, per_row):
    """Out-of-range entries (at or past the count, or below -1) at random valid
    slots of every row; returns the planted picks, the same picks with those
    entries set to -1, and how many were planted."""
    bad, clean = idx.copy(), idx.copy()
    n = 0
    for r in range(idx.shape[0]):
        slots = np.nonzero(idx[r] >= 0)[0]
        pos = rng.choice(slots, min(per_row, len(slots)), replace=False)
        for j, p in enumerate(pos):
            bad[r, p] = counts[r] + j if j % 2 == 0 else -2 - j
            clean[r, p] = -1
            n += 1
    return bad, clean, n


def test_bad_picks_fp8_decode_split(K):
    say("bad picks, FP8 decode")
    B, L, k = 2, [20000, 9001], 512
    layer = S.decode_layer(7070, "csa", B, L, topk=k)
    rng = np.random.default_rng(3)
    N = layer.pool.count
    nv = O.n_visible(layer.tok, layer.m, N)
    sc = rng.standard_normal((B, layer.pool.rows_per_seq))
    idx = O.topk(np.where(np.arange(sc.shape[1])[None] < nv[:, None], sc, -np.inf), nv, k)
    bad, clean, n = plant(idx, N, rng, 9)
    seq = np.arange(B, dtype=np.int32)
    Q = K.QueryRows(dev(seq), dev(layer.tok), dev(layer.pos0), B)
    win, pool, q, sinks = upload_rows(layer.win), upload_rows(layer.pool), tensor_of(layer.q, "bf16"), dev(layer.sinks)

    def run(ix):
        return K.dsv4_sparse_attn(Q, q, win, layer.W, pool, dev(ix), sinks, layer.sm_scale, layer.R, layer.theta,
                                  out_dtype=torch.float32)
    K.dsv4_read_diagnostics(reset=True)
    out_bad = run(bad)
    d_bad = K.dsv4_read_diagnostics(reset=True)
    out_clean = run(clean)
    d_clean = K.dsv4_read_diagnostics(reset=True)
    say("planted", n, "counted", d_bad["bad_picks"], "clean call", d_clean["bad_picks"])
    assert K.lib().dsv4_attn_workspace(B, layer.H, layer.D, layer.W + k) > 0   # the decode call splits its rows
    assert d_bad["bad_picks"] == n and d_clean["bad_picks"] == 0
    assert torch.equal(out_bad, out_clean)


def test_bad_picks_f16_prefill(K):
    say("bad picks, fp16 prefill")
    H, D, R, W, m, k, Sx = 64, 512, 64, 128, 4, 64, 700
    rng = np.random.default_rng(4)
    kv = (1.28 * rng.standard_normal((1, Sx, D))).astype(np.float32)
    win = upload_rows(S.rowset_from_values(kv, "f16", count=[Sx], first_tok=[0]))
    N = Sx // m
    pool = upload_rows(S.rowset_from_values((1.28 * rng.standard_normal((1, N, D))).astype(np.float32), "f16"))
    q = tensor_of(S.bf16_to_f32(S.bf16_bits((1.28 * rng.standard_normal((Sx, H, D))).astype(np.float32))), "bf16")
    n_vis = np.minimum((np.arange(Sx) + 1) // m, N)
    idx = np.full((Sx, k), -1, np.int32)
    for t in range(Sx):
        c = min(k, n_vis[t])
        idx[t, :c] = np.sort(rng.choice(n_vis[t], c, replace=False)) if c else []
    bad, clean, n = plant(idx, np.full(Sx, N), rng, 3)
    Q = K.QueryRows(dev(np.zeros(Sx, np.int32)), dev(np.arange(Sx, dtype=np.int32)), None, 1)
    sinks = dev(rng.standard_normal(H).astype(np.float32))

    def run(ix):
        return K.dsv4_sparse_attn(Q, q, win, W, pool, dev(ix), sinks, 1 / np.sqrt(D), R, 1.6e5,
                                  out_dtype=torch.float32)
    K.dsv4_read_diagnostics(reset=True)
    out_bad = run(bad)
    d_bad = K.dsv4_read_diagnostics(reset=True)
    out_clean = run(clean)
    d_clean = K.dsv4_read_diagnostics(reset=True)
    say("planted", n, "counted", d_bad["bad_picks"])
    assert d_bad["bad_picks"] == n and d_clean["bad_picks"] == 0
    assert torch.equal(out_bad, out_clean)


def test_off_counts_nothing(K):
    say("diagnostics off")
    prev = K.dsv4_set_diagnostics(False)
    try:
        B, L, k = 1, [9001], 256
        layer = S.decode_layer(7071, "csa", B, L, topk=k)
        idx = np.full((B, k), layer.pool.count[0] + 3, np.int32)   # every pick out of range
        Q = K.QueryRows(dev(np.zeros(B, np.int32)), dev(layer.tok), dev(layer.pos0), B)
        K.dsv4_read_diagnostics(reset=True)
        K.dsv4_sparse_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(layer.win), layer.W, upload_rows(layer.pool),
                           dev(idx), dev(layer.sinks), layer.sm_scale, layer.R, layer.theta, out_dtype=torch.float32)
        assert K.dsv4_read_diagnostics(reset=True) == {"ref_raises": 0, "bad_picks": 0}
    finally:
        K.dsv4_set_diagnostics(prev)
