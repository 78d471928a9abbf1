"""Pins of the oracle's storage encoders (quantise-on-write): FP8 E4M3 rows
with an fp32 row scale and BF16 rope channels, and OCP MXFP4 blocks.

The references are independent of the oracle: torch's own float8_e4m3fn and
bfloat16 casts (round to nearest even), the OCP MX E2M1 grid written out, and
exact arithmetic on values chosen to sit on a code or halfway between two."""
import numpy as np
import pytest
import torch

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8r_codes_match_torch_where_the_scale_is_exact(orc):
    """With amax = 448 * 2^k the row scale is the exact power 2^k, so x/s is
    exact and every code must be torch's round-to-nearest-even cast."""
    rng = np.random.default_rng(11)
    for k in (-9, -3, 0, 2):
        x = (rng.standard_normal((64, 448)) * 100.0).astype(np.float32)
        x = np.clip(x, -447.0, 447.0) * np.float32(2.0 ** k)
        x[:, 0] = np.float32(448.0 * 2.0 ** k)           # sets amax
        x[:, 1:20] = np.float32(2.0 ** k) * np.float32(rng.uniform(-0.02, 0.02, (64, 19)))   # subnormal range
        rows, sc = orc.quantize_fp8r(np.concatenate([x, np.zeros((64, 64), np.float32)], 1), 64)
        assert np.all(sc == np.float32(2.0 ** k))
        assert np.array_equal(rows[:, :448], _torch_e4m3(x / sc[:, None]))


def test_fp8r_every_code_and_every_midpoint(orc):
    """Every finite E4M3 magnitude encodes to itself, and the midpoint between
    two neighbours goes to the even code (the scale is 1: amax = 448)."""
    mags = np.array([orc.e4m3_to_f64(c) for c in range(127)])
    vals = np.concatenate([mags, -mags, (mags[:-1] + mags[1:]) / 2, -(mags[:-1] + mags[1:]) / 2]).astype(np.float32)
    n = len(vals)
    x = np.zeros((n, 448 + 64), np.float32)
    x[:, 0] = 448.0
    x[:, 1] = vals
    rows, sc = orc.quantize_fp8r(x, 64)
    assert np.all(sc == 1.0)
    assert np.array_equal(rows[:, 1], _torch_e4m3(vals))
    codes = rows[:127, 1]
    assert np.array_equal(codes, np.arange(127))                      # exact values keep their code
    mid = rows[254:254 + 126, 1]
    assert np.all(mid % 2 == 0)                                       # ties to the even code


def test_fp8r_bf16_tail_matches_torch_and_zero_rows(orc):
    rng = np.random.default_rng(12)
    x = rng.standard_normal((50, 512)).astype(np.float32) * 3
    x[7] = 0.0
    rows, sc = orc.quantize_fp8r(x, 64)
    tail = rows[:, 448:].copy().view(np.uint16)
    ref = torch.from_numpy(x[:, 448:]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tail, ref)
    assert sc[7] == 1.0 and np.all(rows[7, :448] == 0)
    # decode(encode(x)) is within half a code step of x (relative 2^-4 for normals)
    dec = np.array([[orc.e4m3_to_f64(c) for c in r] for r in rows[:5, :448]]) * sc[:5, None]
    err = np.abs(dec - x[:5, :448])
    assert np.all(err <= np.maximum(np.abs(x[:5, :448]) * 2.0 ** -4, sc[:5, None] * 2.0 ** -10) + 1e-12)


def test_mxfp4_grid_scale_ties_and_sign(orc):
    """OCP MX: block scale 2^(floor(log2 amax) - 2); elements on the E2M1 grid
    keep their code, midpoints go to the even code, |x/scale| > 6 saturates,
    and zero never takes the sign bit."""
    # block 0: amax 6 -> scale 2^0; the grid and its midpoints
    mids = (E2M1[:-1] + E2M1[1:]) / 2
    vals = np.concatenate([E2M1, -E2M1[1:], mids, -mids, [-0.0, 6.0]]).astype(np.float32)[:32]
    x = np.zeros((1, 64), np.float32)
    x[0, :len(vals)] = vals
    x[0, 31] = 6.0
    # block 1: amax 13 -> floor(log2 13) = 3 -> scale 2^1; 13/2 = 6.5 saturates to 6
    x[0, 32] = 13.0
    x[0, 33] = -0.1
    nib, sc = orc.quantize_mxfp4(x)
    assert sc[0, 0] == 127 and sc[0, 1] == 128
    codes = np.stack([nib[0] & 15, nib[0] >> 4], 1).reshape(-1)
    for i in range(8):
        assert codes[i] == i                                           # grid values
    for i in range(1, 8):
        assert codes[7 + i] == (8 | i)                                 # negatives
    for j, m in enumerate(mids):                                       # midpoints -> even code
        c = codes[15 + j]
        assert E2M1[c & 7] in (E2M1[j], E2M1[j + 1]) and c % 2 == 0
    assert codes[32] == 7                                              # saturated at 6
    assert codes[33] == 0                                              # -0.05 -> +0, no negative zero


def test_mxfp4_random_blocks_within_half_step(orc):
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((40, 128)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    nib, sc = orc.quantize_mxfp4(x)
    codes = np.stack([nib & 15, nib >> 4], -1).reshape(40, 128)
    scale = np.repeat(2.0 ** (sc.astype(np.int64) - 127), 32, axis=1)
    dec = np.where(codes & 8, -1.0, 1.0) * E2M1[codes & 7] * scale
    amax = np.abs(x.reshape(40, 4, 32)).max(-1)
    assert np.array_equal(sc.astype(np.int64) - 127, np.floor(np.log2(amax)).astype(np.int64) - 2)
    a = np.abs(x) / scale
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    assert np.all(np.abs(dec - x) <= np.maximum(step / 2, a - 6) * scale + 1e-30)
