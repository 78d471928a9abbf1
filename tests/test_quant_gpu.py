"""Quantise-on-write (dsv4_quantize) against the oracle's encoders, bit for bit,
and a decode step over caches written that way."""
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
    return K


def _rows(n, dim, seed):
    """N(0,1) rows over a wide range of magnitudes, an all-zero row, and rows
    holding E4M3 / E2M1 codes and midpoints exactly at scale 1."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, dim)) * np.exp(rng.uniform(-10, 10, (n, 1)))
    x[3] = 0.0
    mags = np.array([O.e4m3_to_f64(c) for c in range(127)])
    vals = np.concatenate([mags, (mags[:-1] + mags[1:]) / 2])
    x[5, : min(dim, len(vals))] = vals[: min(dim, len(vals))]
    x[5, 0] = 448.0
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5, -0.1])
    x[6] = np.resize(np.concatenate([grid, -grid]), dim)
    x[6, ::32] = 6.0
    return x.astype(np.float32)


@pytest.mark.parametrize("dim,tail,xkind", [(512, 64, "f32"), (512, 64, "bf16"), (256, 0, "f16"), (128, 64, "f32")])
def test_quantize_fp8r_bit_exact(K, dim, tail, xkind):
    say("quantize fp8r", dim, tail, xkind)
    x = _rows(333, dim, 21 + dim)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[xkind]
    xt = torch.from_numpy(x).to(tdt).cuda()
    xv = xt.float().cpu().numpy()          # the stored input values, exactly
    rows, sc = K.dsv4_quantize(xt, K.DSV4_FP8R, tail)
    rows_o, sc_o = O.quantize_fp8r(xv, tail)
    torch.cuda.synchronize()
    assert np.array_equal(sc.cpu().numpy(), sc_o)
    assert np.array_equal(rows.cpu().numpy(), rows_o)


@pytest.mark.parametrize("dim,xkind", [(128, "f32"), (512, "bf16"), (64, "f32"), (256, "f16")])
def test_quantize_mxfp4_bit_exact(K, dim, xkind):
    say("quantize mxfp4", dim, xkind)
    x = _rows(257, dim, 31 + dim)
    x[9, :32] = 0.0                       # one all-zero block
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[xkind]
    xt = torch.from_numpy(x).to(tdt).cuda()
    xv = xt.float().cpu().numpy()
    nib, sc = K.dsv4_quantize(xt, K.DSV4_MXFP4)
    nib_o, sc_o = O.quantize_mxfp4(xv)
    torch.cuda.synchronize()
    assert np.array_equal(sc.cpu().numpy(), sc_o)
    assert np.array_equal(nib.cpu().numpy(), nib_o)


def test_decode_over_caches_written_on_the_gpu(K):
    """Pool entries from the compressor and window rows from the rope kernel,
    quantised to FP8 rows on the GPU, then a CSA decode step; the oracle pools,
    rotates and quantises with its own code and attends over its own rows."""
    say("decode over quantised caches")
    rng = np.random.default_rng(41)
    B, L, D, R, m, W, H, k, theta = 2, 4096, 512, 64, 4, 128, 64, 256, 1.6e5
    N = L // m
    c = S.bf16_to_f32(S.bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32)))
    z = S.bf16_to_f32(S.bf16_bits(rng.standard_normal((B, L, D)).astype(np.float32)))
    bias = (0.1 * rng.standard_normal((2 * m, D))).astype(np.float32)
    kv = S.bf16_to_f32(S.bf16_bits(rng.standard_normal((B, W, D)).astype(np.float32)))
    pos0 = np.zeros(B, np.int64)
    wpos = np.arange(L - W, L)
    # GPU: pool (fp32) -> FP8 rows; window rope (fp32) -> FP8 rows
    pool_g = K.dsv4_compress(tensor_of(c, "bf16"), tensor_of(z, "bf16"), dev(bias), m, True, R, theta,
                             pos0=dev(pos0), out_dtype=torch.float32)
    prow, psc = K.dsv4_quantize(pool_g, K.DSV4_FP8R, R)
    kvr_g = torch.stack([K.dsv4_rope(tensor_of(kv[b], "bf16"), dev(wpos), R, theta, out_dtype=torch.float32)
                         for b in range(B)])
    wrow, wsc = K.dsv4_quantize(kvr_g, K.DSV4_FP8R, R)
    cnt = dev(np.full(B, N, np.int32))
    pool_rs = K.RowStore(prow, K.DSV4_FP8R, D, cnt, tail=R, row_scale=psc)
    win_rs = K.RowStore(wrow, K.DSV4_FP8R, D, dev(np.full(B, W, np.int32)), tail=R, row_scale=wsc,
                        first_tok=dev(np.full(B, L - W, np.int32)))
    q = S.bf16_to_f32(S.bf16_bits(rng.standard_normal((B, H, D)).astype(np.float32)))
    idx = np.stack([np.sort(rng.choice(N, k, replace=False)) for _ in range(B)]).astype(np.int32)
    sinks = rng.standard_normal(H).astype(np.float32)
    seq, tok = np.arange(B, dtype=np.int32), np.full(B, L - 1, np.int32)
    Q = K.QueryRows(dev(seq), dev(tok), dev(pos0), B)
    out = K.dsv4_sparse_attn(Q, tensor_of(q, "bf16"), win_rs, W, pool_rs, dev(idx), dev(sinks), 1 / np.sqrt(D), R,
                             theta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # oracle chain on its own values
    pool_o = O.compress(S.bf16_bits(c), S.bf16_bits(z), bias, m, True, R, theta, pos0, kind="bf16")
    prow_o, psc_o = O.quantize_fp8r(pool_o.astype(np.float32), R)
    kvr_o = np.stack([O.rope(kv[b], wpos, R, theta, +1) for b in range(B)])
    wrow_o, wsc_o = O.quantize_fp8r(kvr_o.astype(np.float32), R)
    pool_set = S.RowSet("fp8r", prow_o, D, np.full(B, N, np.int32), tail=R, row_scale=psc_o)
    win_set = S.RowSet("fp8r", wrow_o, D, np.full(B, W, np.int32), tail=R, row_scale=wsc_o,
                       first_tok=np.full(B, L - W, np.int32))
    ref = O.attn(seq, tok, pos0, S.bf16_bits(q), "bf16", win_set, W, pool_set, "csa", idx=idx, sinks=sinks,
                 sm_scale=1 / np.sqrt(D), rope_dim=R, theta=theta)
    # the stored codes agree except where fp32 and fp64 pooling round to neighbouring codes
    same = np.mean(prow.cpu().numpy() == prow_o)
    say("pool codes identical", round(float(same), 5))
    assert same > 0.99
    assert_close(out.cpu().numpy(), ref, "bf16", "decode over GPU-written FP8 caches")
