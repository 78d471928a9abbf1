"""Variable-length batched prefill and the window-only (sliding) layer type.

Several sequences of different lengths share one call: the query rows are the
flat list of (sequence, token) pairs and every per-sequence store carries its
own count (cu_seqlens-style batching).  The window-only layer is the sparse
attention with no compressed branch (top-k 0) and its own rope theta.  Both
are checked against the oracle, which takes the same stored rows."""
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


def _varlen_case(lens, H, D, R, W, m, Hi, Di, theta, seed, rows="f16"):
    """Stores padded to the longest sequence, counts per sequence; q and the
    index inputs as flat [sum(lens), ...] rows in sequence order."""
    rng = np.random.default_rng(seed)
    B, Lmax = len(lens), max(lens)
    r16 = lambda x: S.bf16_to_f32(S.bf16_bits(np.asarray(x, np.float32)))
    kv_rot = np.zeros((B, Lmax, D))
    pool = np.zeros((B, Lmax // m, D))
    keys = np.zeros((B, Lmax // m, Di), np.float32)
    pos0 = np.array([0, 4096, 17][:B], np.int64)
    for b, L in enumerate(lens):
        kv = 1.28 * rng.standard_normal((L, D))
        kv_rot[b, :L] = O.rope(kv, pos0[b] + np.arange(L), R, theta, +1)
        pool[b, : L // m] = 1.28 * rng.standard_normal((L // m, D))
        keys[b, : L // m] = rng.standard_normal((L // m, Di))
    win = S.rowset_from_values(kv_rot.astype(np.float32), rows, count=np.array(lens), first_tok=np.zeros(B))
    pset = S.rowset_from_values(pool.astype(np.float32), rows, count=np.array([L // m for L in lens]))
    kset = S.rowset_from_values(keys, "bf16", count=np.array([L // m for L in lens]))
    seq = np.concatenate([np.full(L, b, np.int32) for b, L in enumerate(lens)])
    tok = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    T = len(seq)
    q = r16(1.28 * rng.standard_normal((T, H, D)))
    q_idx = r16(rng.standard_normal((T, Hi, Di)))
    w = rng.standard_normal((T, Hi)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    return dict(win=win, pool=pset, keys=kset, seq=seq, tok=tok, q=q, q_idx=q_idx, w=w, sinks=sinks, pos0=pos0, B=B)


@pytest.mark.parametrize("lens,k,rows", [
    ([700, 333, 1030], 64, "f16"),
    ([129, 4, 517], 100, "bf16"),
])
def test_varlen_prefill_chain(K, lens, k, rows):
    """Index top-k and sparse attention over a flat batch of sequences of
    different lengths (each with its own pos0, count and pool)."""
    say("varlen prefill", lens, k, rows)
    H, D, R, W, m, Hi, Di, theta = 64, 512, 64, 128, 4, 32, 128, 1.6e5
    c = _varlen_case(lens, H, D, R, W, m, Hi, Di, theta, 900 + sum(lens), rows)
    seq, tok = c["seq"], c["tok"]
    scale = 1.0 / np.sqrt(Hi * Di)
    sc = O.index_scores(seq, tok, S.bf16_bits(c["q_idx"]), "bf16", c["w"], c["keys"], m, scale)
    nv = O.n_visible(tok, m, c["keys"].count[seq])
    idx_o = O.topk(sc, nv, k)
    Q = K.QueryRows(dev(seq), dev(tok), dev(c["pos0"]), c["B"])
    idx = K.dsv4_index_topk(Q, tensor_of(c["q_idx"], "bf16"), dev(c["w"]), upload_rows(c["keys"]), m, k, scale)
    out = K.dsv4_sparse_attn(Q, tensor_of(c["q"], "bf16"), upload_rows(c["win"]), W, upload_rows(c["pool"]),
                             dev(idx_o), dev(c["sinks"]), 1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    say("top-k", check_topk(idx.cpu().numpy(), sc, nv, k, "varlen"))
    ref = O.attn(seq, tok, c["pos0"], S.bf16_bits(c["q"]), "bf16", c["win"], W, c["pool"], "csa", idx=idx_o,
                 sinks=c["sinks"], sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    assert_close(out.cpu().numpy(), ref, "bf16", "varlen sparse attention")


@pytest.mark.parametrize("lens,H,W,rows", [
    ([700, 333, 1030], 64, 128, "f16"),
    ([90, 2, 300], 16, 64, "bf16"),
])
def test_sliding_window_layer(K, lens, H, W, rows):
    """Window-only attention (no compressed branch), rope theta 10000."""
    say("sliding layer", lens, H, W, rows)
    D, R, theta = 512, 64, 1e4
    c = _varlen_case(lens, H, D, R, W, 4, 32, 128, theta, 700 + sum(lens), rows)
    seq, tok = c["seq"], c["tok"]
    Q = K.QueryRows(dev(seq), dev(tok), dev(c["pos0"]), c["B"])
    out = K.dsv4_sparse_attn(Q, tensor_of(c["q"], "bf16"), upload_rows(c["win"]), W, None, None, dev(c["sinks"]),
                             1 / np.sqrt(D), R, theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = O.attn(seq, tok, c["pos0"], S.bf16_bits(c["q"]), "bf16", c["win"], W, None, "csa", idx=None,
                 sinks=c["sinks"], sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    assert_close(out.cpu().numpy(), ref, "bf16", "sliding window attention")
