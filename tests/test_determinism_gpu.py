"""Run-to-run determinism: the same inputs twice give the same bits.

Every reduction on the path has a fixed order (no float atomics; the long-row
top-k adds integer counts with atomics, whose sum does not depend on order),
so two calls on identical inputs must agree bit for bit: the CSA prefill chain
(compressors, rope, indexer, top-k, attention over fp16 rows), and the decode
step over FP8 caches with long rows (level-0 histogram in the scan, candidate
compaction, rows split over several workgroups and merged).  Parity with the
oracle is tested elsewhere; this only fixes that nothing varies between runs.
"""
import numpy as np
import pytest
import torch

import dsv4_synth as S
from gpu_helpers import dev, tensor_of, upload_rows

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


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.uint8).cpu().numpy()


def test_prefill_chain_twice(K):
    say("determinism: CSA prefill chain, S=3000, fp16 rows")
    c = S.flash_prefill(4321, "csa", B=1, S=3000, topk=512, pos0=[0])
    Sx, D, R, m, W, k = c.S, c.D, c.R, c.m, c.W, c.topk
    seq = np.zeros(Sx, np.int32)
    tok = np.arange(Sx, dtype=np.int32)
    Q = K.QueryRows(dev(seq), dev(tok), dev(c.pos0), 1)
    cnt = dev(np.full(1, Sx // m, np.int32))
    args = dict(c=tensor_of(c.c, "bf16"), z=tensor_of(c.z, "bf16"), ci=tensor_of(c.c_idx, "bf16"),
                zi=tensor_of(c.z_idx, "bf16"), kv=tensor_of(c.kv.reshape(Sx, D), "bf16"),
                q=tensor_of(c.q.reshape(Sx, c.H, D), "bf16"), qi=tensor_of(c.q_idx.reshape(Sx, c.Hi, c.Di), "bf16"),
                w=dev(c.w_idx.reshape(Sx, c.Hi)), pos=dev(np.arange(Sx, dtype=np.int64)))

    def run():
        pool = K.dsv4_compress(args["c"], args["z"], dev(c.bias), m, True, R, c.theta, pos0=dev(c.pos0),
                               out_dtype=torch.float16)
        kpool = K.dsv4_compress(args["ci"], args["zi"], dev(c.bias_idx), m, True)
        kv = K.dsv4_rope(args["kv"], args["pos"], R, c.theta, out_dtype=torch.float16)
        idx = K.dsv4_index_topk(Q, args["qi"], args["w"], K.RowStore(kpool, K.DSV4_BF16, c.Di, cnt), m, k,
                                c.score_scale)
        win = K.RowStore(kv.view(1, Sx, D), K.DSV4_F16, D, dev(np.full(1, Sx, np.int32)),
                         first_tok=dev(np.zeros(1, np.int32)))
        out = K.dsv4_sparse_attn(Q, args["q"], win, W, K.RowStore(pool, K.DSV4_F16, D, cnt), idx, dev(c.sinks),
                                 c.sm_scale, R, c.theta)
        torch.cuda.synchronize()
        return [_bits(x) for x in (pool, kpool, kv, idx, out)]

    a, b = run(), run()
    for name, x, y in zip(("pool", "index keys", "window rope", "picks", "attention"), a, b):
        assert np.array_equal(x, y), f"{name} differs between two runs"


@pytest.mark.parametrize("kind,B,L,k", [
    ("csa", 4, [131072, 70001, 4093, 9], 512),
    ("hca", 3, [262144, 70000, 3000], 0),
])
def test_decode_step_twice(K, kind, B, L, k):
    say("determinism: decode step", kind, B, L, k)
    layer = S.decode_layer(91 + B, kind, B, L, topk=max(k, 1))
    seq = np.arange(B, dtype=np.int32)
    Q = K.QueryRows(dev(seq), dev(layer.tok), dev(layer.pos0), B)
    q = tensor_of(layer.q, "bf16")
    win, pool, sinks = upload_rows(layer.win), upload_rows(layer.pool), dev(layer.sinks)

    def run():
        if kind == "csa":
            kp = upload_rows(layer.kpool)
            idx = K.dsv4_index_topk(Q, tensor_of(layer.q_idx, "bf16"), dev(layer.w_idx), kp, layer.m, k,
                                    layer.score_scale)
            out = K.dsv4_sparse_attn(Q, q, win, layer.W, pool, idx, sinks, layer.sm_scale, layer.R, layer.theta)
            res = [idx, out]
        else:
            res = [K.dsv4_hca_attn(Q, q, win, layer.W, pool, layer.m, sinks, layer.sm_scale, layer.R, layer.theta)]
        torch.cuda.synchronize()
        return [_bits(x) for x in res]

    a, b = run(), run()
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), f"{kind} decode output {i} differs between two runs"
