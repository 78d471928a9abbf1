"""The torch packers used for device-side benchmark inputs produce exactly the
bytes of the numpy packers (checked on the CPU)."""
import numpy as np
import torch

import dsv4_synth as S


def test_fp8r_torch_matches_numpy():
    x = np.random.default_rng(0).standard_normal((3, 7, 512)).astype(np.float32)
    a_rows, a_s = S.fp8r_pack(x, 64)
    b_rows, b_s = S.fp8r_pack_torch(torch.from_numpy(x), 64)
    assert np.array_equal(a_rows, b_rows.numpy()) and np.array_equal(a_s, b_s.numpy())


def test_mxfp4_torch_matches_numpy():
    x = np.random.default_rng(1).standard_normal((5, 9, 128)).astype(np.float32)
    x[0, 0, :32] = 0.0
    x[1, 1, 5] = 0.75      # ties between grid points
    x[1, 1, 6] = -2.5
    a_p, a_s = S.mxfp4_pack(x)
    b_p, b_s = S.mxfp4_pack_torch(torch.from_numpy(x))
    assert np.array_equal(a_p, b_p.numpy()) and np.array_equal(a_s, b_s.numpy())


def test_draw_torch_reproducible():
    a = S.draw_torch(3, "q", (4, 5), 2.0, device="cpu")
    b = S.draw_torch(3, "q", (4, 5), 2.0, device="cpu")
    c = S.draw_torch(3, "kv", (4, 5), 2.0, device="cpu")
    assert torch.equal(a, b) and not torch.equal(a, c)


def test_numpy_chunks_regenerate():
    case = S.flash_prefill(5, "csa", B=2, S=40, H=4, D=64, Hi=4, Di=32, topk=4)
    part = S.flash_prefill(5, "csa", B=2, S=40, H=4, D=64, Hi=4, Di=32, topk=4, with_q=False)
    assert np.array_equal(S.prefill_q_rows(part, 1, 3, 17), case.q[1, 3:17])
