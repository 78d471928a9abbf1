"""The CSA attention block from hidden states: every projection through
dsv4_linear, the CSA core, then the grouped low-rank output projection and
o_b, against the oracle's fp64 chain (P1/P2 products, O1 rope, O2 compressor,
O4/O5 indexer, O6 attention).  Both sides keep the activations in the same
storage types (bf16 projections, fp16 K=V rows, fp32 head weights), each
rounding its own values; the attention takes the oracle's index set (the
GPU's own top-k is checked against the oracle's scores with the gap rule).
Small configuration: hidden 256, q_lora 128, 64 heads x 512 (64 rope
channels), indexer 64 x 128, m 4, window 128, top-k 64, 8 groups x 128."""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import assert_close, check_topk, dev, upload_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


def _bf(x):
    return S.bf16_to_f32(S.bf16_bits(np.asarray(x, np.float32)))


def _f16(x):
    return np.asarray(x, np.float32).astype(np.float16).astype(np.float32)


@pytest.mark.parametrize("Sx,pos0", [(300, 0), (523, 4096)])
def test_csa_block(K, Sx, pos0):
    say("csa block", Sx, pos0)
    rng = np.random.default_rng(Sx)
    hid, qlr, H, D, R, Hi, Di, m, W, k, G, olr = 256, 128, 64, 512, 64, 64, 128, 4, 128, 64, 8, 128
    theta = 1.6e5
    N = Sx // m
    x = _bf(rng.standard_normal((Sx, hid)))
    wt = lambda *shape: _bf(0.02 * rng.standard_normal(shape) * np.sqrt(4096 / shape[-1]))
    Wqa, Wqb, Wkv, Wc, Wz = wt(qlr, hid), wt(H * D, qlr), wt(D, hid), wt(D, hid), wt(D, hid)
    WqI, Ww, WcI, WzI = wt(Hi * Di, hid), wt(Hi, hid), wt(Di, hid), wt(Di, hid)
    Woa, Wob = wt(G, olr, H * D // G), wt(hid, G * olr)
    bias = (0.1 * rng.standard_normal((2 * m, D))).astype(np.float32)
    bias_i = (0.1 * rng.standard_normal((2 * m, Di))).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    sm, ss = 1 / np.sqrt(D), 1 / np.sqrt(Hi * Di)
    P0 = np.array([pos0], np.int64)
    seq, tok = np.zeros(Sx, np.int32), np.arange(Sx, dtype=np.int32)

    # ---- oracle chain, its values rounded to the storage types
    qa = _bf(O.linear(x, Wqa))
    q = _bf(O.linear(qa, Wqb)).reshape(Sx, H, D)
    kv = _bf(O.linear(x, Wkv))
    c, z = _bf(O.linear(x, Wc)), _bf(O.linear(x, Wz))
    qI = _bf(O.linear(x, WqI)).reshape(Sx, Hi, Di)
    w = O.linear(x, Ww).astype(np.float32)
    cI, zI = _bf(O.linear(x, WcI)), _bf(O.linear(x, WzI))
    kv_rot = _f16(O.rope(kv, pos0 + np.arange(Sx), R, theta, +1))
    pool = _f16(O.compress(S.bf16_bits(c[None]), S.bf16_bits(z[None]), bias, m, True, R, theta, P0, kind="bf16"))
    kpool = _bf(O.compress(S.bf16_bits(cI[None]), S.bf16_bits(zI[None]), bias_i, m, True, kind="bf16"))
    kp_set = S.rowset_from_values(kpool, "bf16")
    sc_o = O.index_scores(seq, tok, S.bf16_bits(qI), "bf16", w, kp_set, m, ss)
    nv = O.n_visible(tok, m, kp_set.count)
    idx_o = O.topk(sc_o, nv, k)
    win_set = S.rowset_from_values(kv_rot[None], "f16", count=[Sx], first_tok=[0])
    pool_set = S.rowset_from_values(pool, "f16")
    o = _bf(O.attn(seq, tok, P0, S.bf16_bits(q), "bf16", win_set, W, pool_set, "csa", idx=idx_o, sinks=sinks,
                   sm_scale=sm, rope_dim=R, theta=theta))
    oa = _bf(O.grouped_linear(o.reshape(Sx, H * D), Woa))
    y_ref = O.linear(oa, Wob)

    # ---- the same block on the GPU, through the C ABI
    t = lambda a: dev(a, torch.bfloat16)
    lin = K.dsv4_linear
    xd = t(x)
    qa_d = lin(xd, t(Wqa))
    q_d = lin(qa_d, t(Wqb)).view(Sx, H, D)
    kv_d = lin(xd, t(Wkv))
    c_d, z_d = lin(xd, t(Wc)).view(1, Sx, D), lin(xd, t(Wz)).view(1, Sx, D)
    qI_d = lin(xd, t(WqI)).view(Sx, Hi, Di)
    w_d = lin(xd, t(Ww), out_dtype=torch.float32)
    cI_d, zI_d = lin(xd, t(WcI)).view(1, Sx, Di), lin(xd, t(WzI)).view(1, Sx, Di)
    pos0_d = dev(P0)
    kvr_d = K.dsv4_rope(kv_d, dev(pos0 + np.arange(Sx, dtype=np.int64)), R, theta, out_dtype=torch.float16)
    pool_d = K.dsv4_compress(c_d, z_d, dev(bias), m, True, R, theta, pos0=pos0_d, out_dtype=torch.float16)
    kpool_d = K.dsv4_compress(cI_d, zI_d, dev(bias_i), m, True)
    cnt = dev(np.array([N], np.int32))
    Q = K.QueryRows(dev(seq), dev(tok), pos0_d, 1)
    idx_g = K.dsv4_index_topk(Q, qI_d, w_d, K.RowStore(kpool_d, K.DSV4_BF16, Di, cnt), m, k, ss)
    win_rs = K.RowStore(kvr_d.view(1, Sx, D), K.DSV4_F16, D, dev(np.array([Sx], np.int32)),
                        first_tok=dev(np.zeros(1, np.int32)))
    o_d = K.dsv4_sparse_attn(Q, q_d, win_rs, W, K.RowStore(pool_d, K.DSV4_F16, D, cnt), dev(idx_o), dev(sinks),
                             sm, R, theta)
    oa_d = lin(o_d.view(Sx, H * D), t(Woa), groups=G)
    y_d = lin(oa_d, t(Wob), out_dtype=torch.float32)
    torch.cuda.synchronize()

    # the block's own picks: its keys and queries come from GPU products, which
    # round to bf16 where the oracle's do not always, so the end-to-end gap bound
    # applies; on shared stored keys and queries the 1e-5 rule applies
    res = check_topk(idx_g.cpu().numpy(), sc_o, nv, k, "block top-k", gap=1e-3)
    say("top-k rows exact / near-tie", res)
    idx_s = K.dsv4_index_topk(Q, t(qI), dev(w), upload_rows(kp_set), m, k, ss)
    torch.cuda.synchronize()
    say("shared-key top-k", check_topk(idx_s.cpu().numpy(), sc_o, nv, k, "block top-k (shared keys)"))
    assert_close(qa_d.float().cpu().numpy(), qa, "bf16", "q_a")
    assert_close(pool_d.float().cpu().numpy(), pool, "bf16", "pooled K=V entries")
    assert_close(o_d.float().cpu().numpy(), o, "bf16", "attention output")
    assert_close(y_d.cpu().numpy(), y_ref, "bf16", "block output")
