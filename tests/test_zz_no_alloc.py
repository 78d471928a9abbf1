"""The allocation-free index/top-k entry point (dsv4_index_topk_noalloc): its
static scratch replaces the caller's workspace, so its picks and scores must be
the bits dsv4_index_topk gives on the same inputs -- on two calls in a row, the
second smaller (the scratch keeps the first call's contents), over pools short
enough for one workgroup per row and long enough for the radix-threshold passes
whose histograms must start at zero; and in each case the picks pass the
oracle's 1e-5 gap rule."""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import check_topk, dev, tensor_of, upload_rows

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def K():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import compressed_sparse_kv_csa_amd as K
    K.lib()
    return K


def _case(K, seed, kind, B, L, k):
    layer = S.decode_layer(seed, "csa", B, L, topk=k, idx_kind=kind)
    kp = layer.kpool
    seq = np.arange(B, dtype=np.int32)
    tok = layer.tok
    Q = K.QueryRows(dev(seq), dev(tok), None, B)
    if kind == "mxfp4":
        qst, qsc = layer.q_idx_packed, layer.q_idx_scale
        qdev, qscd = dev(qst), dev(qsc)
    else:
        qst, qsc = S.bf16_bits(layer.q_idx), None
        qdev, qscd = tensor_of(layer.q_idx, "bf16"), None
    return layer, kp, seq, tok, Q, qst, qsc, qdev, qscd


@pytest.mark.parametrize("kind,first,second,k", [
    ("bf16", (4, [4 * 40000, 4 * 39000, 4 * 2000, 7]), (2, [4 * 20000, 4 * 17000]), 512),
    ("mxfp4", (3, [4 * 70000, 4 * 65000, 4 * 100]), (1, [4 * 9000]), 1024),
    ("bf16", (5, [4 * 3000] * 5), (2, [4 * 1000, 4 * 900]), 256),
])
def test_noalloc_equals_workspace_call(K, kind, first, second, k):
    for n, (B, L) in enumerate((first, second)):
        say("noalloc", kind, "call", n, "B", B, "L", L, "k", k)
        layer, kp, seq, tok, Q, qst, qsc, qdev, qscd = _case(K, 600 + 7 * n + B, kind, B, L, k)
        kps = upload_rows(kp)
        w = dev(layer.w_idx)
        need = K.lib().dsv4_index_topk_workspace(B, kps.stride, k)
        assert need <= K.NOALLOC_SCRATCH_BYTES
        idx_ws, sc_ws = K.dsv4_index_topk(Q, qdev, w, kps, layer.m, k, layer.score_scale, q_idx_scale=qscd,
                                           want_scores=True)
        idx_na = torch.full((B, k), 12345, dtype=torch.int32, device="cuda")
        sc_na = torch.full((B, k), 7.0, dtype=torch.float32, device="cuda")
        K.dsv4_index_topk_noalloc(Q, qdev, w, kps, layer.m, k, layer.score_scale, idx_na, q_idx_scale=qscd,
                                  score_out=sc_na)
        torch.cuda.synchronize()
        assert torch.equal(idx_na, idx_ws), "picks differ from the workspace call"
        assert torch.equal(sc_na, sc_ws), "pick scores differ from the workspace call"
        ref = O.index_scores(seq, tok, qst, kind, layer.w_idx, kp, layer.m, layer.score_scale, q_scale=qsc)
        nv = O.n_visible(tok, layer.m, kp.count)
        say("gap rule", check_topk(idx_na.cpu().numpy(), ref, nv, k, "noalloc"))


def test_noalloc_rejects_oversize(K):
    """A call whose scratch need exceeds the static array returns
    DSV4_EWORKSPACE and launches nothing (the output keeps its contents)."""
    B, N, k = 36, 1 << 17, 64          # 36 rows x 131072 entries x 4 B = 18 MiB of scores
    assert K.lib().dsv4_index_topk_workspace(B, N, k) > K.NOALLOC_SCRATCH_BYTES
    keys = torch.zeros(B, N, 128, dtype=torch.bfloat16, device="cuda")
    kps = K.RowStore(keys, K.DSV4_BF16, 128, torch.full((B,), N, dtype=torch.int32, device="cuda"))
    Q = K.QueryRows.decode(torch.full((B,), 4 * N, dtype=torch.int32, device="cuda"))
    q = torch.zeros(B, 64, 128, dtype=torch.bfloat16, device="cuda")
    w = torch.ones(B, 64, dtype=torch.float32, device="cuda")
    out = torch.full((B, k), 5, dtype=torch.int32, device="cuda")
    with pytest.raises(K.Dsv4Error) as e:
        K.dsv4_index_topk_noalloc(Q, q, w, kps, 4, k, 1.0, out)
    assert e.value.code == K.DSV4_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 5).all())
