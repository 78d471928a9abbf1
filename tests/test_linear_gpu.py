"""The projections (dsv4_linear) against the oracle's fp64 products: plain and
grouped, ragged M and N (partial tiles), every output type, and the
full-size shapes of the Flash attention block on a sample of output rows."""
import numpy as np
import pytest
import torch

import dsv4_synth as S
import oracle as O
from gpu_helpers import assert_close, dev

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


def _tol_close(got, ref, K_, what):
    """fp32 accumulation of K_ bf16 products of O(1/sqrt(K_))-scaled operands:
    |err| <= K_ * 2^-23 * max|x| max|w| per output, well inside 1e-4 at these
    sizes."""
    assert_close(got, ref, "f32", what)


@pytest.mark.parametrize("M,N,Kd,out", [(1, 16, 64, torch.float32), (300, 200, 192, torch.float32),
                                        (129, 513, 256, torch.bfloat16), (128, 128, 4096, torch.float32),
                                        (37, 11072, 128, torch.float16), (700, 64, 1024, torch.float32),
                                        # 256 x 256 tiles with ragged edges in both dimensions
                                        (1300, 1100, 128, torch.float32), (1030, 2049, 256, torch.bfloat16)])
def test_linear(K, M, N, Kd, out):
    say("linear", M, N, Kd, out)
    rng = np.random.default_rng(M * 7 + N)
    x = _bf(rng.standard_normal((M, Kd)))
    w = _bf(rng.standard_normal((N, Kd)) / np.sqrt(Kd))
    y = K.dsv4_linear(dev(x, torch.bfloat16), dev(w, torch.bfloat16), out_dtype=out)
    torch.cuda.synchronize()
    ref = O.linear(x, w)
    if out == torch.float32:
        _tol_close(y.cpu().numpy(), ref, Kd, "linear")
    else:
        assert_close(y.float().cpu().numpy(), ref, "bf16", "linear (16-bit output)")


def test_linear_grouped(K):
    """The grouped output projection: 8 groups of 8 heads x 512 -> 1024 each."""
    say("grouped linear")
    rng = np.random.default_rng(5)
    M, G, Kd, N = 67, 8, 4096, 1024
    x = _bf(rng.standard_normal((M, G * Kd)))
    w = _bf(rng.standard_normal((G, N, Kd)) / np.sqrt(Kd))
    y = K.dsv4_linear(dev(x, torch.bfloat16), dev(w, torch.bfloat16), out_dtype=torch.float32, groups=G)
    torch.cuda.synchronize()
    _tol_close(y.cpu().numpy(), O.grouped_linear(x, w), Kd, "grouped linear")


def test_linear_strided_rows(K):
    """x rows with a stride wider than K (a column slice of a wider tensor)."""
    say("linear, strided x")
    rng = np.random.default_rng(6)
    full = _bf(rng.standard_normal((90, 640)))
    w = _bf(rng.standard_normal((96, 256)) / 16)
    xt = dev(full, torch.bfloat16)[:, 128:384]
    y = K.dsv4_linear(xt, dev(w, torch.bfloat16), out_dtype=torch.float32)
    torch.cuda.synchronize()
    _tol_close(y.cpu().numpy(), O.linear(full[:, 128:384], w), 256, "strided linear")


def test_linear_fullsize_sampled(K):
    """The Flash block's largest products at T = 8192 rows (q_b 1024 -> 32768,
    o_b 8192 -> 4096) on sampled rows, in the launch configuration the
    benchmark uses."""
    say("linear full size")
    g = torch.Generator(device="cuda").manual_seed(11)
    for (M, N, Kd) in [(8192, 32768, 1024), (8192, 4096, 8192)]:
        x = (torch.randn(M, Kd, device="cuda", generator=g)).to(torch.bfloat16)
        w = (torch.randn(N, Kd, device="cuda", generator=g) / np.sqrt(Kd)).to(torch.bfloat16)
        y = K.dsv4_linear(x, w, out_dtype=torch.float32)
        torch.cuda.synchronize()
        rows = np.random.default_rng(M + N).choice(M, 24, replace=False)
        xs = x[rows].float().cpu().numpy()
        ref = O.linear(xs, w.float().cpu().numpy())
        _tol_close(y[rows].cpu().numpy(), ref, Kd, f"linear {M}x{N}x{Kd}")
        del x, w, y
