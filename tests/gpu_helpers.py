"""Helpers shared by the GPU tests: upload synthetic inputs, run the oracle and
the HIP path on the same data, and the comparison rules.

Comparison rules (from the accuracy targets of the method):
* floating outputs: |gpu - ref| <= atol + rtol * |ref| elementwise, with
  atol = rtol = 1e-4 on fp32 paths and atol 1e-2, rtol 2e-2 on bf16/fp8 paths;
* top-k: the pick set must be exactly min(k, n) distinct visible entries, every
  pick must score >= v_k - 1e-5 and every entry scoring > v_k + 1e-5 must be
  picked, where v_k is the oracle's k-th largest fp64 score (near-ties inside
  the 1e-5 band may resolve either way; outside it the sets are identical).
"""
from __future__ import annotations

import numpy as np
import torch

import dsv4_synth as S
import compressed_sparse_kv_csa_amd as K

TOL = {"f32": (1e-4, 1e-4), "bf16": (1e-2, 2e-2)}
GAP = 1e-5


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def kind_code(kind: str) -> int:
    return {"f32": K.DSV4_F32, "bf16": K.DSV4_BF16, "fp8r": K.DSV4_FP8R, "mxfp4": K.DSV4_MXFP4,
            "f16": K.DSV4_F16}[kind]


def upload_rows(rs: S.RowSet) -> K.RowStore:
    data = rs.data if (rs.data.dtype == np.uint8 and rs.data.ndim == 3) else \
        rs.data.view(np.uint8).reshape(rs.n_seq, rs.rows_per_seq, -1)
    return K.RowStore(
        data=dev(data),
        dtype=kind_code(rs.kind), dim=rs.dim, count=dev(rs.count.astype(np.int32)), tail=rs.tail,
        row_scale=None if rs.row_scale is None else dev(rs.row_scale.astype(np.float32)),
        blk_scale=None if rs.blk_scale is None else dev(rs.blk_scale.astype(np.uint8)),
        first_tok=None if rs.first_tok is None else dev(rs.first_tok.astype(np.int32)))


def tensor_of(x: np.ndarray, store: str) -> torch.Tensor:
    """Device tensor holding stored values (bf16 values are exact in bf16)."""
    return dev(np.asarray(x, np.float32), torch.bfloat16 if store == "bf16" else torch.float32)


def assert_close(gpu: np.ndarray, ref: np.ndarray, store: str, what: str = ""):
    atol, rtol = TOL[store]
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        i = np.unravel_index(np.argmax(err - (atol + rtol * np.abs(ref))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
                             f"(atol {atol}, rtol {rtol}); worst at {i}: gpu {gpu[i]!r} ref {ref[i]!r}; "
                             f"max abs err {err.max():.3e}")


def check_topk(gpu_idx: np.ndarray, scores: np.ndarray, n_valid: np.ndarray, k: int, what: str = "",
               gap: float = None) -> dict:
    """Gap rule.  Returns counts of exact-set rows and near-tie rows."""
    GAP_ = GAP if gap is None else gap
    exact = ties = 0
    for r in range(gpu_idx.shape[0]):
        n = int(n_valid[r])
        kk = min(k, n)
        row = gpu_idx[r]
        picks = row[row >= 0]
        assert np.all(row[len(picks):] == -1), f"{what} row {r}: -1 sentinel not at the tail: {row}"
        assert len(picks) == kk, f"{what} row {r}: {len(picks)} picks, expected {kk}"
        assert len(np.unique(picks)) == kk and np.all(picks < n), f"{what} row {r}: invalid picks"
        if kk == 0:
            exact += 1
            continue
        sc = scores[r, :n]
        order = np.lexsort((np.arange(n), -sc))
        vk = sc[order[kk - 1]]
        assert np.all(sc[picks] >= vk - GAP_), f"{what} row {r}: a pick scores below v_k - gap"
        must = np.nonzero(sc > vk + GAP_)[0]
        assert np.all(np.isin(must, picks)), f"{what} row {r}: a clear winner is missing"
        ref_set = np.sort(order[:kk])
        if np.array_equal(np.sort(picks), ref_set):
            exact += 1
        else:
            ties += 1
    return {"exact": exact, "near_tie": ties}
