"""Decode attention at the largest split counts, against the oracle.

A short batch of long row lists splits each query's rows over nsplit
workgroups (at most 64) whose partials the merge kernel combines; the merge
has instances for split bounds 8, 16, 32 and 64, each for an exact and a
smaller count.  The other parity cases reach at most 32 splits.  These HCA
decode shapes reach 64 (one sequence at a 1M context: 8192 pool entries plus
the window, 260 tiles of 32 rows) and 40 (three sequences, the longest with
4992 entries), on FP8 rows (the decode kernel) and on fp16 rows (the split
path of the prefill kernel).  The split count is read back from the
workspace size the library asks for.
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
    prev = K.dsv4_set_batch_invariant(False)
    yield K
    K.dsv4_set_batch_invariant(prev)


def _nsplit(K, T, H, D, max_rows):
    ws = K.lib().dsv4_attn_workspace(T, H, D, max_rows)
    if ws == 0:
        return 1
    return (ws - 256) // (T * H * (2 * D + 8))


@pytest.mark.parametrize("rows,B,L,ns,out", [
    ("fp8r", 1, [1048576], 64, "f32"),
    ("fp8r", 1, [1048576], 64, "bf16"),
    ("fp8r", 3, [638976, 1000, 70000], 40, "f32"),
    ("f16", 1, [1048576], 64, "f32"),
    ("f16", 3, [638976, 1000, 70000], 40, "f32"),
])
def test_hca_decode_many_splits(K, rows, B, L, ns, out):
    say("hca decode many splits", rows, B, L, ns, out)
    layer = S.decode_layer(300 + B, "hca", B, L)
    D, H, W = layer.D, layer.H, layer.W
    pool, win = layer.pool, layer.win
    if rows == "f16":
        rng = np.random.default_rng(301)
        pool = S.rowset_from_values(rng.standard_normal((B, pool.rows_per_seq, D)).astype(np.float32), "f16",
                                    count=pool.count)
        win = S.rowset_from_values(rng.standard_normal((B, W, D)).astype(np.float32), "f16", count=win.count,
                                   first_tok=win.first_tok)
    assert _nsplit(K, B, H, D, W + pool.rows_per_seq) == ns
    seq = np.arange(B, dtype=np.int32)
    ref = O.attn(seq, layer.tok, layer.pos0, S.bf16_bits(layer.q), "bf16", win, W, pool, "hca", m=layer.m,
                 sinks=layer.sinks, sm_scale=layer.sm_scale, rope_dim=layer.R, theta=layer.theta)
    Q = K.QueryRows(dev(seq), dev(layer.tok), dev(layer.pos0), B)
    got = K.dsv4_hca_attn(Q, tensor_of(layer.q, "bf16"), upload_rows(win), W, upload_rows(pool), layer.m,
                          dev(layer.sinks), layer.sm_scale, layer.R, layer.theta,
                          out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    assert_close(got.float().cpu().numpy(), ref, "bf16", f"hca decode, {rows} rows, {ns} splits, {out} out")
