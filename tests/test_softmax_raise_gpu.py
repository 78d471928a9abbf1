"""The fp16 attention kernels take each head's probabilities against a fixed
reference, the first tile's maximum logit.  When a later tile passes the
reference by more than 15 in log2 units (so no probability could stay inside
fp16's range), the reference is raised inside that tile to the largest logit
seen so far: the partial sums and the accumulators scale by the power of two
between the two references and the tile's probabilities are taken again.
These cases force one and two such raises per query: every query shares a
common direction c, the rows of the first tiles are small noise (logits near
0), and chosen picks are rows along c with natural-log logits of about 12, 22
and 24, placed in successive tiles.  Checked against the oracle's exact
softmax on the fp16 prefill path, the FP8 decode path (split over several
workgroups) and the generic bf16 path, and the number of raises against the
rule run on the CPU.  The test also checks, on the CPU, that the inputs
really take the logit spread past the threshold."""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import assert_close, dev, tensor_of, upload_rows

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


def along(c, logit, D, rng):
    """A row whose dot product with a query c + noise, times 1/sqrt(D), is
    about `logit` (c has norm sqrt(D) over the channels it uses)."""
    return c * (logit / np.sqrt(D)) + 0.02 * rng.standard_normal(D)


@pytest.mark.parametrize("rows,H", [("f16", 64), ("bf16", 64), ("f16", 16)])
def test_prefill_raise(K, rows, H):
    say("prefill reference raise", rows, H)
    D, R, W, theta = 512, 0, 128, 1e4     # no rope channels: logits are plain dot products
    rng = np.random.default_rng(99)
    Sx, m, k = 900, 4, 64
    c = rng.standard_normal(D)
    c *= np.sqrt(D) / np.linalg.norm(c)
    q = S.bf16_to_f32(S.bf16_bits((c + 0.5 * rng.standard_normal((Sx, H, D))).astype(np.float32)))
    N = Sx // m
    pool = 0.02 * rng.standard_normal((N, D))
    jumps = {10: (5, 12.0), 40: (6, 22.0), 50: (7, 24.0)}   # pick position -> (pool entry, logit)
    for e, lg in jumps.values():
        pool[e] = along(c, lg, D, rng)
    win = 0.02 * rng.standard_normal((Sx, D))
    wset = S.rowset_from_values(win[None].astype(np.float32), rows, count=[Sx], first_tok=[0])
    pset = S.rowset_from_values(pool[None].astype(np.float32), rows)
    tok = np.arange(Sx, dtype=np.int32)
    seq = np.zeros(Sx, np.int32)
    n = np.minimum((tok + 1) // m, N)
    idx = np.full((Sx, k), -1, np.int32)
    forced = 0
    for t in range(Sx):
        cnt = min(k, n[t])
        if n[t] >= 8 + k:                  # jump entries at fixed pick positions, the rest from [8, n)
            pick = rng.choice(np.arange(8, n[t]), k, replace=False)
            for pos, (e, _) in jumps.items():
                pick[pos] = e
            idx[t] = pick
            forced += 1
        elif cnt:
            idx[t, :cnt] = rng.choice(np.arange(8, n[t]) if n[t] >= 8 + cnt else n[t], cnt, replace=False)
    assert forced > 300
    # the inputs do what the test is for: for a token with forced picks, the
    # window tiles stay near 0 and the pool tiles jump past the threshold twice
    t = Sx - 1
    s = np.einsum("hd,nd->hn", q[t].astype(np.float64), pool[idx[t]]) / np.sqrt(D) * LOG2E
    first = np.max(np.einsum("hd,nd->hn", q[t].astype(np.float64), win[t - W + 1:t - W + 33]) / np.sqrt(D) * LOG2E, 1)
    assert np.all(s[:, :32].max(1) > first + 15.5)
    assert np.all(s[:, 32:].max(1) > s[:, :32].max(1) + 15.5)
    sinks = rng.standard_normal(H).astype(np.float32)
    Q = K.QueryRows(dev(seq), dev(tok), None, 1)
    prev = K.dsv4_set_diagnostics(True)
    try:
        K.dsv4_read_diagnostics(reset=True)
        out = K.dsv4_sparse_attn(Q, tensor_of(q, "bf16"), upload_rows(wset), W, upload_rows(pset), dev(idx),
                                 dev(sinks), 1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
        diag = K.dsv4_read_diagnostics(reset=True)
    finally:
        K.dsv4_set_diagnostics(prev)
    ref = O.attn(seq, tok, np.zeros(1, np.int64), S.bf16_bits(q), "bf16", wset, W, pset, "csa", idx=idx,
                 sinks=sinks, sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    assert_close(out.cpu().numpy(), ref, "bf16", "attention across softmax reference raises")
    # the raise counter against the rule run on the CPU over every query whose
    # picks hold a jump entry (the others' logits stay near 0): thresholds a
    # little either side of 15 bound the fp16 rounding of q~ and the rows
    lo = hi = 0
    jump_rows = {e for e, _ in jumps.values()}
    for t in range(Sx):
        if not jump_rows & set(idx[t][idx[t] >= 0].tolist()):
            continue
        rows_t = np.concatenate([win[max(0, t - W + 1):t + 1], pool[idx[t][idx[t] >= 0]]])
        lg = q[t].astype(np.float64) @ rows_t.T / np.sqrt(D) * LOG2E
        lo += count_raises(lg, 15.05)
        hi += count_raises(lg, 14.95)
    say("reference raises", diag["ref_raises"], "expected", lo, "..", hi)
    if rows == "f16":   # the fixed-reference kernels: every 16-head block raises at least once per forced query
        assert lo >= forced * (H // 16) and lo <= diag["ref_raises"] <= hi
    else:               # the generic kernel keeps a running maximum: it never raises
        assert diag["ref_raises"] == 0
    assert diag["bad_picks"] == 0


def count_raises(lg, thr, group=16):
    """The fixed-reference rule on one query's logits (heads x rows, log2
    units, rows in list order), per block of `group` heads (the heads one wave
    scores): 32-row tiles; the first tile's maximum is each head's reference; a
    tile whose maximum passes a reference of the block by more than thr raises
    every reference of that block to its head's largest logit seen so far."""
    count = 0
    for h0 in range(0, lg.shape[0], group):
        blk = lg[h0:h0 + group]
        ref, seen = None, np.full(blk.shape[0], -np.inf)
        for a in range(0, blk.shape[1], 32):
            m = blk[:, a:a + 32].max(1)
            seen = np.maximum(seen, m)
            if ref is None:
                ref = m.copy()
            elif np.any(m > ref + thr):
                count += 1
                ref = seen.copy()
    return count


def test_decode_raise_fp8_split(K):
    say("decode reference raise, FP8 rows, split")
    D, R, W, H, k, theta = 512, 64, 128, 64, 512, 1.6e5
    rng = np.random.default_rng(98)
    B, L = 3, 8000
    N = L // 4
    c = rng.standard_normal(D)
    c[D - R:] = 0                          # rope turns the last 64 channels: keep the jump off them
    c *= np.sqrt(D) / np.linalg.norm(c)
    q = S.bf16_to_f32(S.bf16_bits((c + 0.5 * rng.standard_normal((B, H, D))).astype(np.float32)))
    pools = 0.02 * rng.standard_normal((B, N, D))
    wins = 0.02 * rng.standard_normal((B, W, D))
    idx = np.empty((B, k), np.int32)
    for b in range(B):
        pick = rng.choice(np.arange(8, N), k, replace=False)
        # raises in the pool tiles near the end of the list, and in the middle
        for pos, e, lg in ((200, 2, 12.0), (300, 3, 22.0), (505, 4, 24.0)):
            pools[b, e] = along(c, lg, D, rng)
            pick[pos] = e
        idx[b] = pick
    pset = S.rowset_from_values(pools.astype(np.float32), "fp8r", tail=R)
    wset = S.rowset_from_values(wins.astype(np.float32), "fp8r", tail=R, count=np.full(B, W),
                                first_tok=np.full(B, L - W))
    sinks = rng.standard_normal(H).astype(np.float32)
    seq, tok = np.arange(B, dtype=np.int32), np.full(B, L - 1, np.int32)
    Q = K.QueryRows(dev(seq), dev(tok), dev(np.zeros(B, np.int64)), B)
    out = K.dsv4_sparse_attn(Q, tensor_of(q, "bf16"), upload_rows(wset), W, upload_rows(pset), dev(idx),
                             dev(sinks), 1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.attn(seq, tok, np.zeros(B, np.int64), S.bf16_bits(q), "bf16", wset, W, pset, "csa", idx=idx,
                 sinks=sinks, sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    assert_close(out.cpu().numpy(), ref, "bf16", "FP8 decode across softmax reference raises")
