"""Batch invariance: a query row's outputs must not depend on the other rows of
the call (DeepSeek-V4 review page, "Muon and MoE system": bitwise-identical
results for a token whatever its batch).  Each case computes a batch, then a
subset of its rows (in another order) as a batch of its own, and requires equal
bits.  Attention needs dsv4_set_batch_invariant(1) (otherwise short batches are
split over their rows); indexer scores and top-k are invariant in either mode,
including across the many-query and few-query scoring kernels.  Every output of
the invariant mode is also compared with the oracle: equal bits alone would let
a wrong but deterministic kernel pass."""
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
    prev = K.dsv4_set_batch_invariant(True)
    yield K
    K.dsv4_set_batch_invariant(prev)


def _subset_rows(n, rng):
    pick = rng.choice(n, 5, replace=False)
    return pick[::-1].copy()          # another order as well as a smaller batch


def test_decode_attention_invariant(K):
    say("decode attention, FP8 rows")
    B, L, k = 12, [5000] * 12, 256
    layer = S.decode_layer(4242, "csa", B, L, topk=k)
    rng = np.random.default_rng(1)
    idx = np.stack([np.sort(rng.choice(L[0] // 4, k, replace=False)) for _ in range(B)]).astype(np.int32)
    win, pool = upload_rows(layer.win), upload_rows(layer.pool)
    q, sinks = tensor_of(layer.q, "bf16"), dev(layer.sinks)
    seq = np.arange(B, dtype=np.int32)

    def run(rows):
        Q = K.QueryRows(dev(seq[rows]), dev(layer.tok[rows]), dev(layer.pos0), B)
        return K.dsv4_sparse_attn(Q, q[rows].contiguous(), win, layer.W, pool, dev(idx[rows]), sinks,
                                  layer.sm_scale, layer.R, layer.theta, out_dtype=torch.float32)
    full = run(np.arange(B))
    sub_rows = _subset_rows(B, rng)
    sub = run(sub_rows)
    torch.cuda.synchronize()
    assert torch.equal(full[torch.from_numpy(sub_rows).cuda()], sub)
    ref = O.attn(seq, layer.tok, layer.pos0, S.bf16_bits(layer.q), "bf16", layer.win, layer.W, layer.pool, "csa",
                 idx=idx, sinks=layer.sinks, sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
    assert_close(full.cpu().numpy(), ref, "bf16", "invariant-mode FP8 decode attention")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_long_fp8_hca_decode_invariant(K, out_dtype):
    """FP8 HCA decode over long pools with one workgroup per query (no split):
    70000 tokens -> 546 entries + 128 window rows (21 tiles), 64 heads."""
    say("long FP8 HCA decode, invariant mode", out_dtype)
    B = 3
    L = [70000, 70000 - 130, 40001]
    layer = S.decode_layer(4343, "hca", B, L)
    win, pool = upload_rows(layer.win), upload_rows(layer.pool)
    q, sinks = tensor_of(layer.q, "bf16"), dev(layer.sinks)
    seq = np.arange(B, dtype=np.int32)

    def run(rows):
        Q = K.QueryRows(dev(seq[rows]), dev(layer.tok[rows]), dev(layer.pos0), B)
        return K.dsv4_hca_attn(Q, q[rows].contiguous(), win, layer.W, pool, layer.m, sinks, layer.sm_scale,
                               layer.R, layer.theta, out_dtype=out_dtype)
    full = run(np.arange(B))
    sub_rows = np.array([2, 0])
    sub = run(sub_rows)
    torch.cuda.synchronize()
    assert torch.equal(full[torch.from_numpy(sub_rows).cuda()], sub)
    ref = O.attn(seq, layer.tok, layer.pos0, S.bf16_bits(layer.q), "bf16", layer.win, layer.W, layer.pool, "hca",
                 m=layer.m, sinks=layer.sinks, sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
    assert_close(full.float().cpu().numpy(), ref, "bf16", "invariant-mode long FP8 HCA decode")


def test_prefill_attention_invariant(K):
    say("prefill attention, fp16 rows")
    H, D, R, W, m, k, Sx = 64, 512, 64, 128, 4, 64, 1100
    rng = np.random.default_rng(2)
    kv = (1.28 * rng.standard_normal((1, Sx, D))).astype(np.float32)
    win = upload_rows(S.rowset_from_values(kv, "f16", count=[Sx], first_tok=[0]))
    pool_vals = (1.28 * rng.standard_normal((1, Sx // m, D))).astype(np.float32)
    pool = upload_rows(S.rowset_from_values(pool_vals, "f16"))
    q_vals = S.bf16_to_f32(S.bf16_bits((1.28 * rng.standard_normal((Sx, H, D))).astype(np.float32)))
    q = tensor_of(q_vals, "bf16")
    n = np.minimum((np.arange(Sx) + 1) // m, Sx // m)
    idx = np.full((Sx, k), -1, np.int32)
    for t in range(Sx):
        c = min(k, n[t])
        idx[t, :c] = np.sort(rng.choice(n[t], c, replace=False)) if c else []
    sinks_h = rng.standard_normal(H).astype(np.float32)
    sinks = dev(sinks_h)
    tok = np.arange(Sx, dtype=np.int32)

    def run(rows):
        Q = K.QueryRows(dev(np.zeros(len(rows), np.int32)), dev(tok[rows]), None, 1)
        return K.dsv4_sparse_attn(Q, q[rows].contiguous(), win, W, pool, dev(idx[rows]), sinks, 1 / np.sqrt(D), R,
                                  1.6e5, out_dtype=torch.float32)
    full = run(np.arange(Sx))
    sub_rows = np.array([Sx - 1, 700, 3, 129, 555])
    sub = run(sub_rows)
    torch.cuda.synchronize()
    assert torch.equal(full[torch.from_numpy(sub_rows).cuda()], sub)
    chk = np.concatenate([sub_rows, np.arange(0, Sx, 97)])
    win_set = S.rowset_from_values(kv, "f16", count=[Sx], first_tok=[0])
    pool_set = S.rowset_from_values(pool_vals, "f16")
    ref = O.attn(np.zeros(len(chk), np.int32), tok[chk], np.zeros(1, np.int64), S.bf16_bits(q_vals[chk]), "bf16",
                 win_set, W, pool_set, "csa", idx=idx[chk], sinks=sinks_h, sm_scale=1 / np.sqrt(D), rope_dim=R,
                 theta=1.6e5)
    assert_close(full[torch.from_numpy(chk).cuda()].cpu().numpy(), ref, "bf16", "invariant-mode prefill attention")


def test_indexer_invariant(K):
    """2100 query rows take the many-query scoring kernel; 4 of them alone take
    the per-query kernel: scores and picks must agree bit for bit."""
    say("indexer scores and top-k")
    Hi, Di, m, k, Sx = 64, 128, 4, 64, 2100
    rng = np.random.default_rng(3)
    keys = rng.standard_normal((1, Sx // m, Di)).astype(np.float32)
    kp = upload_rows(S.rowset_from_values(keys, "bf16"))
    q_vals = S.bf16_to_f32(S.bf16_bits(rng.standard_normal((Sx, Hi, Di)).astype(np.float32)))
    q_idx = tensor_of(q_vals, "bf16")
    w_h = rng.standard_normal((Sx, Hi)).astype(np.float32)
    w = dev(w_h)
    tok = np.arange(Sx, dtype=np.int32)
    scale = 1 / np.sqrt(Hi * Di)

    def run(rows):
        Q = K.QueryRows(dev(np.zeros(len(rows), np.int32)), dev(tok[rows]), None, 1)
        return K.dsv4_index_topk(Q, q_idx[rows].contiguous(), w[rows].contiguous(), kp, m, k, scale, want_scores=True)
    idx_f, sc_f = run(np.arange(Sx))
    sub_rows = np.array([Sx - 1, 2000, 1024, 77])
    idx_s, sc_s = run(sub_rows)
    torch.cuda.synchronize()
    r = torch.from_numpy(sub_rows).cuda()
    assert torch.equal(idx_f[r], idx_s)
    assert torch.equal(sc_f[r], sc_s)
    chk = np.concatenate([sub_rows, np.arange(3, Sx, 61)])
    kp_set = S.rowset_from_values(keys, "bf16")
    ref = O.index_scores(np.zeros(len(chk), np.int32), tok[chk], S.bf16_bits(q_vals[chk]), "bf16", w_h[chk], kp_set,
                         m, scale)
    nv = O.n_visible(tok[chk], m, kp_set.count[0])
    say("invariant-mode picks", check_topk(idx_f[torch.from_numpy(chk).cuda()].cpu().numpy(), ref, nv, k,
                                           "invariant-mode indexer"))
