"""Benchmark of the CSA/HCA attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-legs] [--no-cpu] [--legs-only]

Default workload: the Flash-shaped CSA layer prefill (batch 1, seq 8192, 64 q
heads x 512 with one shared K=V head, m=4, window 128, indexer 64 x 128, top-k
512).  One step is every stage of the path on that input: KV compressor,
indexer-key compressor, window rope, indexer scores + top-k, sparse attention.
`value` is prefill tokens/s over the K timed steps.  The steps are timed as
HIP graph replays (each step captured once per rotated input copy, so the
kernels of a step run back to back without launch gaps; every graph's output
is checked bit for bit against an eager step); --no-graph times eager launches.

The JSON line also carries
  roofline     -- the dominant kernel (the sparse attention kernel): algorithmic
                  MFMA flops per launch / its mean launch time (HIP events on the
                  launch stream) against the MI355X dense fp16/bf16 peak;
  cpu_baseline -- the fp64 oracle on a bounded sample of query rows of the same
                  workload, on the host cores, scaled to tokens/s;
  legs         -- the other workloads (HCA prefill S=65536, CSA decode 32 x 131072,
                  1M-token mixed CSA+HCA decode), a few steps each.
Inputs are seeded synthetic tensors drawn on the device (dsv4_synth).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA/HCA prefill tokens/s + decode attn GB/s at 1M ctx, % of roofline"
PEAK_MFMA_F16 = 2500.0      # TFLOP/s, dense fp16/bf16 MFMA, MI355X
PEAK_HBM = 8000.0           # GB/s, MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic(summary, key="traffic_bytes_per_launch"):
    """HBM bytes per launch of a kernel (or of one call's kernels, `key`) from
    its committed rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE runs
    scaled by a plain copy's counts), or None when the summary is missing or
    the kernels' sources changed since the counters were taken (sha256 of the
    listed source files)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    try:
        kv = dict(ln.split(": ", 1) for ln in open(path).read().splitlines() if ": " in ln and not ln.startswith(" "))
        h = hashlib.sha256()
        for f in kv["source_files"].split():
            h.update(open(os.path.join(ROOT, "compressed_sparse_kv_csa_amd", "csrc", f), "rb").read())
        if h.hexdigest() != kv["source_sha256"].strip():
            return None
        return int(float(kv[key]))
    except (OSError, KeyError, ValueError):
        return None


# ----------------------------------------------------------------------------- accounting
def csa_prefill_counts(S, m, W, k, H, D, Hi, Di):
    t = np.arange(S, dtype=np.int64)
    n = np.minimum(S // m, (t + 1) // m)
    win = np.minimum(W, t + 1)
    sel = np.minimum(k, n)
    # a row with at most k visible entries picks all of them: it is not scored
    scored = n[n > k]
    return {
        "attn_pairs": int((win + sel).sum()),
        "attn_flop": float((win + sel).sum()) * H * D * 4,
        "index_pairs": int(scored.sum()),
        "index_flop": float(scored.sum()) * Hi * Di * 2,
    }


def hca_prefill_counts(S, m, W, H, D):
    t = np.arange(S, dtype=np.int64)
    n = np.minimum(S // m, (t + 1) // m)
    win = np.minimum(W, t + 1)
    return {"attn_pairs": int((win + n).sum()), "attn_flop": float((win + n).sum()) * H * D * 4}


# ----------------------------------------------------------------------------- workloads
class CsaPrefill:
    """Flash-shaped CSA layer prefill (batch 1, seq 8192, bf16)."""
    name = "flash_csa_prefill_S8192"
    dom_kernel = "k_attn_f16<"
    dom_desc = "k_attn_f16 (fp16 MFMA, fp32 accumulate)"
    stats_summary = "csa_prefill_S8192_kernel_stats.txt"
    hbm_summary = "k_attn_f16_csa_prefill_S8192_hbm.txt"

    def __init__(self, torch, K, S_, seed=1002, S=8192, H=64, D=512, R=64, W=128, Hi=64, Di=128, k=512, m=4):
        self.torch, self.K = torch, K
        bf = torch.bfloat16
        std = S_.ACT_STD
        self.S, self.H, self.D, self.R, self.W, self.Hi, self.Di, self.k, self.m = S, H, D, R, W, Hi, Di, k, m
        self.theta = 160000.0
        self.sm_scale = 1.0 / np.sqrt(D)
        self.score_scale = 1.0 / np.sqrt(Hi * Di)
        dr = lambda name, shape, s=std, dt=bf: S_.draw_torch(seed, name, shape, s, dt)
        self.q = dr("q", (S, H, D))
        self.kv = dr("kv", (S, D))
        self.c = dr("c", (1, S, D))
        self.z = dr("z", (1, S, D))
        self.bias = dr("bias", (2 * m, D), 0.1, None)
        self.q_idx = dr("q_idx", (S, Hi, Di))
        self.w = dr("w_idx", (S, Hi), std, None)
        self.c_idx = dr("c_idx", (1, S, Di))
        self.z_idx = dr("z_idx", (1, S, Di))
        self.bias_idx = dr("bias_idx", (2 * m, Di), 0.1, None)
        self.sinks = dr("sinks", (H,), 1.0, None)
        dev = self.q.device
        self.pos0 = torch.zeros(1, dtype=torch.int64, device=dev)
        self.pos = torch.arange(S, dtype=torch.int64, device=dev)
        self.Q = K.QueryRows.prefill(1, S, self.pos0)
        N = S // m
        f16 = torch.float16   # K=V rows feed the fp16 matrix-core path straight from HBM
        self.pool = torch.empty(1, N, D, dtype=f16, device=dev)
        self.kpool = torch.empty(1, N, Di, dtype=bf, device=dev)
        self.kv_rot = torch.empty(1, S, D, dtype=f16, device=dev)
        self.idx = torch.empty(S, k, dtype=torch.int32, device=dev)
        self.out = torch.empty(S, H, D, dtype=bf, device=dev)
        cnt = torch.full((1,), N, dtype=torch.int32, device=dev)
        self.win_rows = K.RowStore(self.kv_rot, K.DSV4_F16, D, torch.full((1,), S, dtype=torch.int32, device=dev),
                                   first_tok=torch.zeros(1, dtype=torch.int32, device=dev))
        self.pool_rows = K.RowStore(self.pool, K.DSV4_F16, D, cnt)
        self.kpool_rows = K.RowStore(self.kpool, K.DSV4_BF16, Di, cnt)
        self.ws_idx = K.index_topk_workspace(S, N, k, dev)
        self.ws_attn = K.attn_workspace(S, H, D, W + k, dev)
        self.counts = csa_prefill_counts(S, m, W, k, H, D, Hi, Di)

    def step(self, ev=None):
        K, m = self.K, self.m
        K.dsv4_compress(self.c, self.z, self.bias, m, True, self.R, self.theta, pos0=self.pos0, out=self.pool)
        K.dsv4_compress(self.c_idx, self.z_idx, self.bias_idx, m, True, out=self.kpool)
        K.dsv4_rope(self.kv, self.pos, self.R, self.theta, out=self.kv_rot.view(self.S, self.D))
        K.dsv4_index_topk(self.Q, self.q_idx, self.w, self.kpool_rows, m, self.k, self.score_scale, ws=self.ws_idx,
                          out=self.idx)
        if ev is not None:
            ev[0].record()
        K.dsv4_sparse_attn(self.Q, self.q, self.win_rows, self.W, self.pool_rows, self.idx, self.sinks,
                           self.sm_scale, self.R, self.theta, ws=self.ws_attn, out=self.out)
        if ev is not None:
            ev[1].record()

    def tokens(self):
        return self.S


class CsaPrefillSkewed(CsaPrefill):
    """The CSA prefill step with the compressor's candidate input scaled by
    POOL_SCALE: the pooled K=V rows (a convex combination of the candidates) get
    logits far above the window rows', so the attention's fixed softmax
    reference, taken from a query's first (window) tile, is passed by more than
    2^15, repeatedly, and raised inside the tile each time.  Ordinary finite
    inputs (pool values of a few tens); measures what those raises cost."""
    name = "flash_csa_prefill_S8192_skewed_pool"
    POOL_SCALE = 16.0

    def __init__(self, torch, K, S_, **kw):
        super().__init__(torch, K, S_, **kw)
        self.c = (self.c.float() * self.POOL_SCALE).to(self.c.dtype)


class HcaPrefill:
    """Flash-shaped HCA layer prefill (batch 1, seq 65536, m'=128, bf16)."""
    name = "flash_hca_prefill_S65536"
    dom_kernel = "k_attn_f16<"
    dom_desc = "k_attn_f16 (fp16 MFMA, fp32 accumulate)"
    stats_summary = "hca_prefill_S65536_kernel_stats.txt"
    hbm_summary = "k_attn_f16_hca_prefill_S65536_hbm.txt"

    def __init__(self, torch, K, S_, seed=1003, S=65536, H=64, D=512, R=64, W=128, m=128):
        self.torch, self.K = torch, K
        bf = torch.bfloat16
        std = S_.ACT_STD
        self.S, self.H, self.D, self.R, self.W, self.m = S, H, D, R, W, m
        self.theta = 160000.0
        self.sm_scale = 1.0 / np.sqrt(D)
        dr = lambda name, shape, s=std, dt=bf: S_.draw_torch(seed, name, shape, s, dt)
        self.q = dr("q", (S, H, D))
        self.kv = dr("kv", (S, D))
        self.c = dr("c", (1, S, D))
        self.z = dr("z", (1, S, D))
        self.bias = dr("bias", (m, D), 0.1, None)
        self.sinks = dr("sinks", (H,), 1.0, None)
        dev = self.q.device
        self.pos0 = torch.zeros(1, dtype=torch.int64, device=dev)
        self.pos = torch.arange(S, dtype=torch.int64, device=dev)
        self.Q = K.QueryRows.prefill(1, S, self.pos0)
        N = S // m
        f16 = torch.float16
        self.pool = torch.empty(1, N, D, dtype=f16, device=dev)
        self.kv_rot = torch.empty(1, S, D, dtype=f16, device=dev)
        self.out = torch.empty(S, H, D, dtype=bf, device=dev)
        self.win_rows = K.RowStore(self.kv_rot, K.DSV4_F16, D, torch.full((1,), S, dtype=torch.int32, device=dev),
                                   first_tok=torch.zeros(1, dtype=torch.int32, device=dev))
        self.pool_rows = K.RowStore(self.pool, K.DSV4_F16, D, torch.full((1,), N, dtype=torch.int32, device=dev))
        self.ws_attn = K.attn_workspace(S, H, D, W + N, dev)
        self.counts = hca_prefill_counts(S, m, W, H, D)

    def step(self, ev=None):
        K = self.K
        K.dsv4_compress(self.c, self.z, self.bias, self.m, False, self.R, self.theta, pos0=self.pos0, out=self.pool)
        K.dsv4_rope(self.kv, self.pos, self.R, self.theta, out=self.kv_rot.view(self.S, self.D))
        if ev is not None:
            ev[0].record()
        K.dsv4_hca_attn(self.Q, self.q, self.win_rows, self.W, self.pool_rows, self.m, self.sinks, self.sm_scale,
                        self.R, self.theta, ws=self.ws_attn, out=self.out)
        if ev is not None:
            ev[1].record()

    def tokens(self):
        return self.S


def _fp8_store(torch, K, S_, seed, name, B, n, D, R, count, first_tok=None):
    """N(0,1) rows drawn per sequence, stored as FP8 E4M3 (+bf16 rope channels, row scale)."""
    rows, scales = [], []
    for b in range(B):
        x = S_.draw_torch(seed, f"{name}{b}", (n, D), 1.0)
        r, s = S_.fp8r_pack_torch(x, R)
        rows.append(r)
        scales.append(s)
        del x
    return K.RowStore(torch.stack(rows), K.DSV4_FP8R, D, count, tail=R, row_scale=torch.stack(scales),
                      first_tok=first_tok)


class CsaDecode:
    """CSA decode: 32 sequences x 1 query at 131072 tokens (32768 FP8 entries, bf16
    indexer keys, window 128, top-k 512)."""
    name = "csa_decode_B32_L131072"
    hbm_summary = "k_attn_dec_csa_decode_B32_L131072_hbm.txt"

    def __init__(self, torch, K, S_, seed=1004, B=32, L=131072, H=64, D=512, R=64, W=128, Hi=64, Di=128, k=512,
                 m=4, copies=3):
        self.torch, self.K = torch, K
        self.B, self.L, self.H, self.D, self.R, self.W, self.Hi, self.Di, self.k, self.m = B, L, H, D, R, W, Hi, Di, k, m
        self.theta = 160000.0
        self.sm_scale = 1.0 / np.sqrt(D)
        self.score_scale = 1.0 / np.sqrt(Hi * Di)
        N = L // m
        dev = torch.device("cuda")
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        self.Q = K.QueryRows.decode(lens, torch.zeros(B, dtype=torch.int64, device=dev))
        cnt = torch.full((B,), N, dtype=torch.int32, device=dev)
        wcnt = torch.full((B,), W, dtype=torch.int32, device=dev)
        ft = torch.full((B,), L - W, dtype=torch.int32, device=dev)
        self.sets = []
        for cpy in range(copies):   # rotated copies: the step's bytes come from HBM, not the 256 MB MALL
            sd = seed + 100 * cpy
            pool = _fp8_store(torch, K, S_, sd, "pool", B, N, D, R, cnt)
            win = _fp8_store(torch, K, S_, sd, "win", B, W, D, R, wcnt, ft)
            keys = S_.draw_torch(sd, "kpool", (B, N, Di), 1.0, torch.bfloat16)
            kp = K.RowStore(keys, K.DSV4_BF16, Di, cnt)
            q = S_.draw_torch(sd, "q", (B, H, D), 1.0, torch.bfloat16)
            q_idx = S_.draw_torch(sd, "q_idx", (B, Hi, Di), 1.0, torch.bfloat16)
            w = S_.draw_torch(sd, "w_idx", (B, Hi), 1.0)
            sinks = S_.draw_torch(sd, "sinks", (H,), 1.0)
            self.sets.append((pool, win, kp, q, q_idx, w, sinks))
        self.idx = torch.empty(B, k, dtype=torch.int32, device=dev)
        self.out = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.ws_idx = K.index_topk_workspace(B, N, k, dev)
        self.ws_attn = K.attn_workspace(B, H, D, W + k, dev)
        self.i = 0
        row = (D - R) + 2 * R + 4
        self.bytes = {"index_keys": B * N * Di * 2, "gather": B * k * row, "window": B * W * row,
                      "q_o": B * H * D * 2 * 2 + B * Hi * Di * 2 + B * Hi * 4}
        self.bytes["total"] = sum(self.bytes.values())

    def step(self, ev=None):
        K = self.K
        pool, win, kp, q, q_idx, w, sinks = self.sets[self.i % len(self.sets)]
        self.i += 1
        if ev is not None:
            ev[0].record()
        K.dsv4_index_topk(self.Q, q_idx, w, kp, self.m, self.k, self.score_scale, ws=self.ws_idx, out=self.idx)
        if ev is not None:
            ev[1].record()
        K.dsv4_sparse_attn(self.Q, q, win, self.W, pool, self.idx, sinks, self.sm_scale, self.R, self.theta,
                           ws=self.ws_attn, out=self.out)

    def attn_calls(self):
        """The step's attention launches (on the last step's inputs and picks):
        [(name, callable, algorithmic bytes, split partial bytes)]."""
        K = self.K
        pool, win, kp, q, q_idx, w, sinks = self.sets[(self.i - 1) % len(self.sets)]
        row = (self.D - self.R) + 2 * self.R + 4
        alg = self.B * (self.k + self.W) * row + 2 * self.B * self.H * self.D * 2 + self.B * self.k * 4
        f = lambda: K.dsv4_sparse_attn(self.Q, q, win, self.W, pool, self.idx, sinks, self.sm_scale, self.R,
                                       self.theta, ws=self.ws_attn, out=self.out)
        return [("csa_attn", f, alg, _partial_bytes(K, self.B, self.H, self.D, self.W + self.k))]


def _partial_bytes(K, T, H, D, max_rows):
    """Bytes of split partials written and read back by the merge (0 without splits)."""
    ws = K.lib().dsv4_attn_workspace(T, H, D, max_rows)
    return 0 if ws == 0 else 2 * (ws - 256)


class MixedDecode:
    """1M-token mixed decode: 8 sequences at 1,048,576 tokens; one CSA layer (m=4,
    top-k 1024, MXFP4 indexer keys/queries, FP8 KV) + one HCA layer (m'=128, 8192
    FP8 entries, dense), window 128 each."""
    name = "mixed_decode_B8_L1048576"
    hbm_summary = "k_attn_dec_mixed_decode_B8_L1048576_hbm.txt"

    def __init__(self, torch, K, S_, seed=1005, B=8, L=1048576, H=64, D=512, R=64, W=128, Hi=64, Di=128, k=1024,
                 copies=3):
        self.torch, self.K = torch, K
        self.B, self.L, self.H, self.D, self.R, self.W, self.Hi, self.Di, self.k = B, L, H, D, R, W, Hi, Di, k
        self.theta = 160000.0
        self.sm_scale = 1.0 / np.sqrt(D)
        self.score_scale = 1.0 / np.sqrt(Hi * Di)
        N, Nh = L // 4, L // 128
        dev = torch.device("cuda")
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        self.Q = K.QueryRows.decode(lens, torch.zeros(B, dtype=torch.int64, device=dev))
        cnt = torch.full((B,), N, dtype=torch.int32, device=dev)
        cnth = torch.full((B,), Nh, dtype=torch.int32, device=dev)
        wcnt = torch.full((B,), W, dtype=torch.int32, device=dev)
        ft = torch.full((B,), L - W, dtype=torch.int32, device=dev)
        self.sets = []
        for cpy in range(copies):
            sd = seed + 100 * cpy
            pool = _fp8_store(torch, K, S_, sd, "pool", B, N, D, R, cnt)
            win = _fp8_store(torch, K, S_, sd, "win", B, W, D, R, wcnt, ft)
            kps, kss = [], []
            for b in range(B):
                pk, sc = S_.mxfp4_pack_torch(S_.draw_torch(sd, f"kpool{b}", (N, Di), 1.0))
                kps.append(pk)
                kss.append(sc)
            kp = K.RowStore(torch.stack(kps), K.DSV4_MXFP4, Di, cnt, blk_scale=torch.stack(kss))
            qpk, qsc = S_.mxfp4_pack_torch(S_.draw_torch(sd, "q_idx", (B, Hi, Di), 1.0))
            q = S_.draw_torch(sd, "q", (B, H, D), 1.0, torch.bfloat16)
            w = S_.draw_torch(sd, "w_idx", (B, Hi), 1.0)
            sinks = S_.draw_torch(sd, "sinks", (H,), 1.0)
            hpool = _fp8_store(torch, K, S_, sd, "hpool", B, Nh, D, R, cnth)
            hwin = _fp8_store(torch, K, S_, sd, "hwin", B, W, D, R, wcnt, ft)
            hq = S_.draw_torch(sd, "hq", (B, H, D), 1.0, torch.bfloat16)
            hsinks = S_.draw_torch(sd, "hsinks", (H,), 1.0)
            self.sets.append((pool, win, kp, qpk, qsc, q, w, sinks, hpool, hwin, hq, hsinks))
        self.idx = torch.empty(B, k, dtype=torch.int32, device=dev)
        self.out = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.hout = torch.empty(B, H, D, dtype=torch.bfloat16, device=dev)
        self.ws_idx = K.index_topk_workspace(B, N, k, dev)
        self.ws_attn = K.attn_workspace(B, H, D, W + k, dev)
        self.ws_hca = K.attn_workspace(B, H, D, W + Nh, dev)
        self.i = 0
        row = (D - R) + 2 * R + 4
        self.bytes = {"index_keys": B * N * (Di // 2 + Di // 32), "hca_pool": B * Nh * row, "gather": B * k * row,
                      "windows": 2 * B * W * row, "q_o": 2 * B * H * D * 2 * 2 + B * Hi * (Di // 2 + Di // 32) + B * Hi * 4}
        self.bytes["total"] = sum(self.bytes.values())

    def step(self, ev=None):
        K = self.K
        pool, win, kp, qpk, qsc, q, w, sinks, hpool, hwin, hq, hsinks = self.sets[self.i % len(self.sets)]
        self.i += 1
        if ev is not None:
            ev[0].record()
        K.dsv4_index_topk(self.Q, qpk, w, kp, 4, self.k, self.score_scale, q_idx_scale=qsc, ws=self.ws_idx,
                          out=self.idx)
        if ev is not None:
            ev[1].record()
        K.dsv4_sparse_attn(self.Q, q, win, self.W, pool, self.idx, sinks, self.sm_scale, self.R, self.theta,
                           ws=self.ws_attn, out=self.out)
        K.dsv4_hca_attn(self.Q, hq, hwin, self.W, hpool, 128, hsinks, self.sm_scale, self.R, self.theta,
                        ws=self.ws_hca, out=self.hout)

    def attn_calls(self):
        """The step's attention launches: [(name, callable, algorithmic bytes, split partial bytes)]."""
        K = self.K
        pool, win, kp, qpk, qsc, q, w, sinks, hpool, hwin, hq, hsinks = self.sets[(self.i - 1) % len(self.sets)]
        row = (self.D - self.R) + 2 * self.R + 4
        qo = 2 * self.B * self.H * self.D * 2
        Nh = self.L // 128
        csa = lambda: K.dsv4_sparse_attn(self.Q, q, win, self.W, pool, self.idx, sinks, self.sm_scale, self.R,
                                         self.theta, ws=self.ws_attn, out=self.out)
        hca = lambda: K.dsv4_hca_attn(self.Q, hq, hwin, self.W, hpool, 128, hsinks, self.sm_scale, self.R,
                                      self.theta, ws=self.ws_hca, out=self.hout)
        return [("csa_attn", csa, self.B * (self.k + self.W) * row + qo + self.B * self.k * 4,
                 _partial_bytes(K, self.B, self.H, self.D, self.W + self.k)),
                ("hca_attn", hca, self.B * (Nh + self.W) * row + qo,
                 _partial_bytes(K, self.B, self.H, self.D, self.W + Nh))]


class CsaBlock(CsaPrefill):
    """The Flash CSA attention block from hidden states (batch 1, seq 8192):
    the projections (low-rank q 4096 -> 1024 -> 64 x 512, kv, compressor and
    indexer projections from x) as dsv4_linear products, the CSA core as in
    CsaPrefill, then the grouped low-rank output projection (8 groups of
    8 heads x 512 -> 1024 each) and o_b (8192 -> 4096).  x ~ N(0, 1), weights
    ~ N(0, 0.02^2) (the config's initializer range), all bf16."""
    name = "flash_csa_block_S8192"

    def __init__(self, torch, K, S_, seed=1006, S=8192, hidden=4096, q_lora=1024, o_groups=8, o_lora=1024, **kw):
        super().__init__(torch, K, S_, S=S, **kw)
        bf = torch.bfloat16
        H, D, Hi, Di = self.H, self.D, self.Hi, self.Di
        dr = lambda name, shape, s: S_.draw_torch(seed, name, shape, s, bf)
        self.hidden, self.o_groups, self.o_lora = hidden, o_groups, o_lora
        self.x = dr("x", (S, hidden), 1.0)
        ws = 0.02
        self.Wqa = dr("W_qa", (q_lora, hidden), ws)
        self.Wqb = dr("W_qb", (H * D, q_lora), ws)
        self.Wkv = dr("W_kv", (D, hidden), ws)
        self.Wc = dr("W_c", (D, hidden), ws)
        self.Wz = dr("W_z", (D, hidden), ws)
        self.WqI = dr("W_qI", (Hi * Di, hidden), ws)
        self.Ww = dr("W_w", (Hi, hidden), ws)
        self.WcI = dr("W_cI", (Di, hidden), ws)
        self.WzI = dr("W_zI", (Di, hidden), ws)
        self.Woa = dr("W_oa", (o_groups, o_lora, H * D // o_groups), ws)
        self.Wob = dr("W_ob", (hidden, o_groups * o_lora), ws)
        dev = self.x.device
        self.qa = torch.empty(S, q_lora, dtype=bf, device=dev)
        self.oa = torch.empty(S, o_groups * o_lora, dtype=bf, device=dev)
        self.y = torch.empty(S, hidden, dtype=bf, device=dev)
        Hg = H * D // o_groups
        self.gemm_flop = 2 * S * (hidden * (q_lora + 3 * D + Hi * Di + Hi + 2 * Di) + q_lora * H * D
                                  + o_groups * o_lora * Hg + o_groups * o_lora * hidden)
        self.qb_flop = 2 * S * q_lora * H * D

    def step(self, ev=None):
        K, S = self.K, self.S
        lin = K.dsv4_linear
        lin(self.x, self.Wqa, out=self.qa)
        if ev is not None:
            ev[0].record()
        lin(self.qa, self.Wqb, out=self.q.view(S, -1))
        if ev is not None:
            ev[1].record()
        lin(self.x, self.Wkv, out=self.kv)
        lin(self.x, self.Wc, out=self.c.view(S, -1))
        lin(self.x, self.Wz, out=self.z.view(S, -1))
        lin(self.x, self.WqI, out=self.q_idx.view(S, -1))
        lin(self.x, self.Ww, out=self.w)
        lin(self.x, self.WcI, out=self.c_idx.view(S, -1))
        lin(self.x, self.WzI, out=self.z_idx.view(S, -1))
        super().step()
        lin(self.out.view(S, -1), self.Woa, groups=self.o_groups, out=self.oa)
        lin(self.oa, self.Wob, out=self.y)


WORKLOADS = {"csa_prefill": CsaPrefill, "hca_prefill": HcaPrefill, "csa_decode": CsaDecode,
             "mixed_decode": MixedDecode, "csa_block": CsaBlock, "csa_prefill_skewed": CsaPrefillSkewed}


def time_steps(torch, wl, steps, warmup):
    """W untimed steps, then exactly K steps between two synchronisations; the
    dominant kernel is bracketed with events on the launch stream every step
    (the library launches on torch's current stream, which the events see)."""
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern = [a.elapsed_time(b) for a, b in evs]
    return (t1 - t0) * 1e3 / steps, float(np.mean(kern)), float(np.median(kern)), kern


def decode_attn_roofline(torch, wl, reps=10):
    """Each attention launch of a decode step timed alone (HIP events on the
    launch stream; split merge included) against the HBM peak: algorithmic
    bytes (gathered and window rows with their scales, q in, o out, picks) and
    the split partials the merge writes and reads back, reported apart."""
    wl.step()
    torch.cuda.synchronize()
    out = {}
    for name, call, alg, part in wl.attn_calls():
        call()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            call()
            b.record()
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in ev]
        ms = float(np.median(t))
        out[name] = {"ms_median": round(ms, 4), "algorithmic_bytes": int(alg), "GB_per_s": round(alg / ms / 1e6, 1),
                     "frac_hbm_peak": round(alg / ms / 1e6 / PEAK_HBM, 4), "split_partial_bytes": int(part),
                     "GB_per_s_with_partials": round((alg + part) / ms / 1e6, 1),
                     "traffic": measured_traffic(wl.hbm_summary, f"traffic_bytes_per_launch_{name}")}
    return {"attention": out}


def pcts(xs):
    """p10 / p50 / p90 of a list of per-step milliseconds."""
    a = np.asarray(xs, dtype=np.float64)
    return {"p10": round(float(np.percentile(a, 10)), 4), "p50": round(float(np.percentile(a, 50)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def platform_info(torch):
    """ROCm / HIP versions and the GPU's shader clock levels (sysfs), for the record."""
    info = {"device": torch.cuda.get_device_name(0), "hip": getattr(torch.version, "hip", None),
            "torch": torch.__version__}
    try:
        info["rocm"] = open("/opt/rocm/.info/version").read().strip()
    except OSError:
        info["rocm"] = None
    try:
        import glob
        for f in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
            lv = [ln.split(":", 1)[1].strip() for ln in open(f).read().splitlines() if ":" in ln]
            if lv:
                info["sclk_levels"] = lv
                info["sclk_max_mhz"] = max(int("".join(ch for ch in x.split("Mhz")[0] if ch.isdigit()) or 0)
                                           for x in lv)
                break
    except (OSError, ValueError):
        pass
    return info


def profile_kernel_us(summary, kernel_prefix):
    """Average duration (us) of a kernel in a committed rocprofv3 kernel-trace
    summary, or None when the summary is missing, names no such kernel, or the
    kernel's sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    try:
        text = open(path).read()
        kv = dict(ln.split(": ", 1) for ln in text.splitlines() if ": " in ln and not ln.startswith(" "))
        if "source_files" in kv:
            h = hashlib.sha256()
            for f in kv["source_files"].split():
                h.update(open(os.path.join(ROOT, "compressed_sparse_kv_csa_amd", "csrc", f), "rb").read())
            if h.hexdigest() != kv["source_sha256"].strip():
                return None
        else:
            return None
        for ln in text.splitlines():
            parts = ln.split()
            if len(parts) >= 6 and kernel_prefix in ln and parts[0].isdigit():
                return float(parts[1])
    except (OSError, KeyError, ValueError):
        return None
    return None


def _outputs(wl):
    return [t for t in (getattr(wl, "out", None), getattr(wl, "hout", None), getattr(wl, "idx", None)) if t is not None]


def time_steps_graph(torch, wl, steps, warmup):
    """The step captured as HIP graphs (one per rotated input copy) and replayed:
    no launch gaps between the step's kernels.  Every graph's last replay is
    checked bit for bit against an eager step on the same inputs.  Returns
    ms/step, or None when capture is not possible here."""
    n = len(getattr(wl, "sets", [None]))
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(n):
                wl.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        if hasattr(wl, "i"):
            wl.i = 0
        for _ in range(n):   # graph j replays input copy j (wl.step() rotates)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                wl.step()
            graphs.append(g)
        torch.cuda.synchronize()
    except Exception as e:   # noqa: BLE001 - report and fall back to eager timing
        log("graph capture unavailable:", repr(e))
        return None, None
    for i in range(warmup):
        graphs[i % n].replay()
    torch.cuda.synchronize()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        marks[i].record()
        graphs[i % n].replay()
    marks[steps].record()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    per_step = [marks[i].elapsed_time(marks[i + 1]) for i in range(steps)]
    for j in range(n):
        graphs[j].replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in _outputs(wl)]
        if hasattr(wl, "i"):
            wl.i = j
        wl.step()
        torch.cuda.synchronize()
        for a, b in zip(got, _outputs(wl)):
            assert torch.equal(a, b), "graph replay differs from the eager step"
    del graphs
    return ms, per_step


# ----------------------------------------------------------------------------- CPU baseline
def cpu_baseline_csa_prefill(torch, wl, target_s=12.0):
    """The fp64 oracle on a bounded sample of query rows of the same CSA prefill
    input: both compressors and the window rope over the whole sequence (shared
    work), then indexer + top-k + attention for sampled rows; the per-row cost is
    scaled to the full sequence."""
    import dsv4_synth as S_
    import oracle as O
    O.build()
    b16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    S, m, R, th = wl.S, wl.m, wl.R, wl.theta
    c, z, ci, zi = b16(wl.c), b16(wl.z), b16(wl.c_idx), b16(wl.z_idx)
    kv = S_.bf16_to_f32(b16(wl.kv))
    bias, bias_i = wl.bias.cpu().numpy(), wl.bias_idx.cpu().numpy()
    sinks = wl.sinks.cpu().numpy()
    t0 = time.perf_counter()
    pool = O.compress(c, z, bias, m, True, R, th, np.zeros(1, np.int64), kind="bf16")
    kpool = O.compress(ci, zi, bias_i, m, True, kind="bf16")
    kv_rot = O.rope(kv, np.arange(S), R, th, +1)
    t_shared = time.perf_counter() - t0

    def f64rows(x, first_tok=None):
        x = np.ascontiguousarray(x, np.float64)
        return S_.RowSet("f64", x.view(np.uint8).reshape(1, x.shape[1], -1), x.shape[2],
                         np.array([x.shape[1]], np.int32),
                         first_tok=None if first_tok is None else np.array([first_tok], np.int32))
    kp_rows, pool_rows, win_rows = f64rows(kpool), f64rows(pool), f64rows(kv_rot[None], 0)

    def run_rows(rows):
        rows = np.asarray(rows, np.int32)
        n = len(rows)
        qi = b16(wl.q_idx[rows])
        w = wl.w[rows].cpu().numpy()
        q = b16(wl.q[rows])
        seq = np.zeros(n, np.int32)
        t1 = time.perf_counter()
        sc = O.index_scores(seq, rows, qi, "bf16", w, kp_rows, m, wl.score_scale)
        nv = O.n_visible(rows, m, S // m)
        idx = O.topk(sc, nv, wl.k)
        O.attn(seq, rows, np.zeros(1, np.int64), q, "bf16", win_rows, wl.W, pool_rows, "csa", idx=idx, sinks=sinks,
               sm_scale=wl.sm_scale, rope_dim=R, theta=th)
        return time.perf_counter() - t1

    rng = np.random.default_rng(7)
    probe = np.sort(rng.choice(S, 32, replace=False))
    t_probe = run_rows(probe)
    n = int(np.clip(32 * max(1.0, (target_s - t_shared) / max(t_probe, 1e-3)), 32, S))
    sample = np.sort(rng.choice(S, n, replace=False))
    t_rows = run_rows(sample)
    per_row = t_rows / n
    est = t_shared + per_row * S
    # one host thread: a smaller sample of the same rows
    nthr = O.num_threads()
    O.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        O.compress(c, z, bias, m, True, R, th, np.zeros(1, np.int64), kind="bf16")
        O.compress(ci, zi, bias_i, m, True, kind="bf16")
        O.rope(kv, np.arange(S), R, th, +1)
        t_shared1 = time.perf_counter() - t0
        n1 = 48
        t_rows1 = run_rows(np.sort(rng.choice(S, n1, replace=False)))
    finally:
        O.set_num_threads(nthr)
    est1 = t_shared1 + t_rows1 / n1 * S
    return {"value": S / est, "unit": "tokens/s", "cores": nthr, "kind": "oracle",
            "sample": (f"fp64 oracle: both compressors + window rope over all {S} tokens ({t_shared:.2f} s), then "
                       f"indexer + top-k + attention for {n} random query rows ({t_rows:.2f} s), per-row cost "
                       f"scaled to {S} rows"),
            "extrapolated": n < S,
            "value_1thread": round(S / est1, 2), "extrapolated_1thread": True,
            "sample_1thread": f"{n1} random rows on one thread ({t_rows1:.2f} s), shared work {t_shared1:.2f} s",
            "cpu_model": cpu_model(), "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
            "seconds": round(t_shared + t_rows + t_probe + t_shared1 + t_rows1, 2)}


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _host_rows(torch, S_, rs, b, kind):
    """Sequence b of a device RowStore as a one-sequence host RowSet."""
    data = rs.data[b:b + 1].contiguous().view(torch.uint8).cpu().numpy().reshape(1, rs.stride, -1)
    pick = lambda t: None if t is None else t[b:b + 1].cpu().numpy()
    return S_.RowSet(kind, data, rs.dim, rs.count[b:b + 1].cpu().numpy().astype(np.int32), tail=rs.tail,
                     row_scale=pick(rs.row_scale), blk_scale=pick(rs.blk_scale),
                     first_tok=pick(rs.first_tok) if rs.first_tok is not None else None)


def cpu_baseline_decode(torch, wl):
    """The fp64 oracle on one sequence of a decode step (its whole indexer scan,
    top-k and attention; for the mixed step also the HCA layer), scaled to the
    step's B sequences: step time and effective GB/s of the step's algorithmic
    bytes."""
    import dsv4_synth as S_
    import oracle as O
    O.build()
    b16 = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    mixed = isinstance(wl, MixedDecode)
    st = wl.sets[0]
    b = 0
    tok = np.array([wl.L - 1], np.int32)
    seq = np.zeros(1, np.int32)
    p0 = np.zeros(1, np.int64)
    if mixed:
        pool, win, kp, qpk, qsc, q, w, sinks, hpool, hwin, hq, hsinks = st
        m, kind = 4, "mxfp4"
        qi, qis = qpk[b:b + 1].cpu().numpy(), qsc[b:b + 1].cpu().numpy()
    else:
        pool, win, kp, q, q_idx, w, sinks = st
        m, kind = wl.m, "bf16"
        qi, qis = b16(q_idx[b:b + 1]), None
    kp_h = _host_rows(torch, S_, kp, b, kind)
    pool_h, win_h = _host_rows(torch, S_, pool, b, "fp8r"), _host_rows(torch, S_, win, b, "fp8r")
    t0 = time.perf_counter()
    sc = O.index_scores(seq, tok, qi, kind, w[b:b + 1].cpu().numpy(), kp_h, m, wl.score_scale, q_scale=qis)
    nv = O.n_visible(tok, m, kp_h.count)
    idx = O.topk(sc, nv, wl.k)
    t1 = time.perf_counter()
    O.attn(seq, tok, p0, b16(q[b:b + 1]), "bf16", win_h, wl.W, pool_h, "csa", idx=idx, sinks=sinks.cpu().numpy(),
           sm_scale=wl.sm_scale, rope_dim=wl.R, theta=wl.theta)
    t2 = time.perf_counter()
    t_hca = 0.0
    if mixed:
        hpool_h, hwin_h = _host_rows(torch, S_, hpool, b, "fp8r"), _host_rows(torch, S_, hwin, b, "fp8r")
        t3 = time.perf_counter()
        O.attn(seq, tok, p0, b16(hq[b:b + 1]), "bf16", hwin_h, wl.W, hpool_h, "hca", m=128,
               sinks=hsinks.cpu().numpy(), sm_scale=wl.sm_scale, rope_dim=wl.R, theta=wl.theta)
        t_hca = time.perf_counter() - t3
    per_seq = (t1 - t0) + (t2 - t1) + t_hca
    step_s = per_seq * wl.B
    return {"value": round(wl.bytes["total"] / step_s / 1e9, 3), "unit": "GB/s", "cores": O.num_threads(),
            "kind": "oracle", "extrapolated": True, "step_ms": round(step_s * 1e3, 1),
            "sample": (f"fp64 oracle on sequence 0 of {wl.B}: indexer scan + top-k {t1 - t0:.2f} s, CSA attention "
                       f"{t2 - t1:.2f} s" + (f", HCA attention {t_hca:.2f} s" if mixed else "") +
                       f"; scaled to {wl.B} sequences"),
            "cpu_model": cpu_model()}


# ----------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="csa_prefill", choices=sorted(WORKLOADS))
    ap.add_argument("--no-legs", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--leg-steps", type=int, default=5)
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, copy 1 GiB device-to-device once (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the path is "
              f"per-GPU work with no collectives -- run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import compressed_sparse_kv_csa_amd as K
    import dsv4_synth as S_
    assert torch.cuda.is_available(), "bench.py needs the GPU"
    K.lib()

    log("building workload", args.workload)
    wl = WORKLOADS[args.workload](torch, K, S_)
    torch.cuda.synchronize()
    log("timing", args.steps, "steps after", args.warmup, "warmup")
    ms, kern_ms, kern_med, kern_all = time_steps(torch, wl, args.steps, args.warmup)
    log(f"eager: ms/step {ms:.3f}; dominant kernel mean {kern_ms:.3f} ms")
    ms_eager, timing, per_step = ms, "eager launches", None
    if not args.no_graph:
        gms, per_step = time_steps_graph(torch, wl, args.steps, args.warmup)
        if gms is not None:
            ms, timing = gms, "HIP graph replay (outputs checked against an eager step)"
            log(f"graph: ms/step {ms:.3f}")
    rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded, device-drawn N(0,1.28^2) activations)",
           "timing": timing, "ms_per_step_eager": round(ms_eager, 4)}
    if per_step:
        rec["ms_per_step_replays"] = pcts(per_step)
    rec["platform"] = platform_info(torch)
    if isinstance(wl, CsaBlock):
        rec["value"] = round(wl.tokens() / (ms / 1e3), 1)
        rec["unit"] = "tokens/s"
        ach = wl.qb_flop / (kern_ms / 1e3) / 1e12
        rec["roofline"] = {"bound": "mfma", "kernel": "k_linear (q_b projection, bf16 MFMA, fp32 accumulate)",
                           "achieved": round(ach, 2), "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                           "frac": round(ach / PEAK_MFMA_F16, 4), "traffic": None,
                           "algorithmic": f"{wl.qb_flop / 1e9:.1f} GFLOP per launch (8192 x 32768 x 1024 x 2)",
                           "kernel_ms_mean": round(kern_ms, 4), "kernel_ms_median": round(kern_med, 4)}
        rec["config"] = {"workload": wl.name, "seq_len": wl.S, "hidden": wl.hidden, "heads": wl.H,
                         "head_dim": wl.D, "o_groups": wl.o_groups, "o_lora_rank": wl.o_lora,
                         "projection_gflop": round(wl.gemm_flop / 1e9, 1)}
    elif isinstance(wl, (CsaPrefill, HcaPrefill)):
        rec["value"] = round(wl.tokens() / (ms / 1e3), 1)
        rec["unit"] = "tokens/s"
        flop = wl.counts["attn_flop"]
        ach = flop / (kern_ms / 1e3) / 1e12
        traffic = measured_traffic(wl.hbm_summary)
        rec["roofline"] = {"bound": "mfma", "kernel": wl.dom_desc,
                           "achieved": round(ach, 2), "peak": PEAK_MFMA_F16, "unit": "TFLOP/s",
                           "frac": round(ach / PEAK_MFMA_F16, 4), "traffic": traffic,
                           "algorithmic": f"{flop / 1e9:.1f} GFLOP per launch ({wl.counts['attn_pairs']} query-row "
                                          f"pairs x 64 heads x 512 x 4)",
                           "kernel_ms_mean": round(kern_ms, 4), "kernel_ms_median": round(kern_med, 4),
                           "kernel_ms_events": pcts(kern_all)}
        prof_us = profile_kernel_us(wl.stats_summary, wl.dom_kernel)
        if prof_us:
            pa = flop / (prof_us / 1e6) / 1e12
            rec["roofline"].update({"kernel_us_profile": prof_us, "achieved_profile": round(pa, 2),
                                    "frac_profile": round(pa / PEAK_MFMA_F16, 4),
                                    "profile": "profiles/" + wl.stats_summary})
        rec["config"] = {"workload": wl.name, "seq_len": wl.S, "heads": wl.H, "head_dim": wl.D,
                         "window": wl.W, "m": wl.m}
        if isinstance(wl, CsaPrefill):
            rec["config"].update({"topk": wl.k, "index_heads": wl.Hi, "index_dim": wl.Di})
    else:
        gbs = wl.bytes["total"] / (ms / 1e3) / 1e9
        rec["value"] = round(gbs, 1)
        rec["unit"] = "GB/s"
        kb = wl.bytes["index_keys"]
        ach = kb / (kern_ms / 1e3) / 1e9
        rec["roofline"] = {"bound": "hbm", "kernel": "dsv4_index_topk (key scan + top-k)", "achieved": round(ach, 1),
                           "peak": PEAK_HBM, "unit": "GB/s", "frac": round(ach / PEAK_HBM, 4),
                           "traffic": measured_traffic(wl.hbm_summary, "traffic_bytes_per_launch_index_topk"),
                           "kernel_ms_mean": round(kern_ms, 4), "kernel_ms_events": pcts(kern_all)}
        rec["config"] = {"workload": wl.name, "bytes_per_step": wl.bytes}
        if not args.no_cpu:
            log("cpu baseline (oracle, one sequence of the decode step)")
            rec["cpu_baseline"] = cpu_baseline_decode(torch, wl)
    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        rec["copy_probe_bytes"] = 1 << 30
        del src, dst
    if not args.no_cpu and isinstance(wl, CsaPrefill):
        log("cpu baseline (oracle on a sample)")
        rec["cpu_baseline"] = cpu_baseline_csa_prefill(torch, wl)
    if not args.no_legs and args.workload == "csa_prefill":
        legs = {}
        del wl
        torch.cuda.empty_cache()
        for name in ("hca_prefill", "csa_decode", "mixed_decode", "csa_block", "csa_prefill_skewed"):
            log("leg", name)
            lw = WORKLOADS[name](torch, K, S_)
            torch.cuda.synchronize()
            lms, lk, _, _ = time_steps(torch, lw, args.leg_steps, 2)
            lper = None
            if not args.no_graph:
                gms, lper = time_steps_graph(torch, lw, args.leg_steps, 2)
                lms = gms if gms is not None else lms
            if isinstance(lw, CsaBlock):
                ach = lw.qb_flop / (lk / 1e3) / 1e12
                tot = (lw.gemm_flop + lw.counts["attn_flop"] + lw.counts.get("index_flop", 0)) / (lms / 1e3) / 1e12
                legs[name] = {"workload": lw.name, "tokens_per_s": round(lw.tokens() / (lms / 1e3), 1),
                              "ms_per_step": round(lms, 3), "block_tflops": round(tot, 1),
                              "projection_gflop": round(lw.gemm_flop / 1e9, 1),
                              "q_b_gemm_ms": round(lk, 3), "q_b_gemm_tflops": round(ach, 1),
                              "q_b_gemm_frac_mfma_peak": round(ach / PEAK_MFMA_F16, 4)}
            elif isinstance(lw, CsaPrefillSkewed):
                prev = K.dsv4_set_diagnostics(True)
                try:
                    K.dsv4_read_diagnostics(reset=True)
                    lw.step()
                    diag = K.dsv4_read_diagnostics(reset=True)
                finally:
                    K.dsv4_set_diagnostics(prev)
                legs[name] = {"workload": lw.name, "pool_value_scale": lw.POOL_SCALE,
                              "tokens_per_s": round(lw.tokens() / (lms / 1e3), 1), "ms_per_step": round(lms, 3),
                              "softmax_ref_raises": diag["ref_raises"],
                              "ref_raises_per_query": round(diag["ref_raises"] / lw.tokens(), 3),
                              "attn_kernel_ms": round(lk, 3), "attn_kernel_ms_unskewed": round(kern_ms, 3),
                              "raise_cost": round(lk / kern_ms - 1.0, 3)}
            elif isinstance(lw, HcaPrefill):
                ach = lw.counts["attn_flop"] / (lk / 1e3) / 1e12
                legs[name] = {"workload": lw.name, "tokens_per_s": round(lw.tokens() / (lms / 1e3), 1),
                              "ms_per_step": round(lms, 3), "attn_kernel_ms": round(lk, 3),
                              "attn_tflops": round(ach, 1), "attn_frac_mfma_peak": round(ach / PEAK_MFMA_F16, 4)}
            else:
                gbs = lw.bytes["total"] / (lms / 1e3) / 1e9
                ik = lw.bytes["index_keys"] / (lk / 1e3) / 1e9
                legs[name] = {"workload": lw.name, "GB_per_s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM, 4),
                              "ms_per_step": round(lms, 4), "bytes_per_step": lw.bytes["total"],
                              "index_topk_ms": round(lk, 4), "index_scan_GB_per_s": round(ik, 1)}
                legs[name].update(decode_attn_roofline(torch, lw))
                if not args.no_cpu:
                    legs[name]["cpu_baseline"] = cpu_baseline_decode(torch, lw)
            if lper:
                legs[name]["ms_per_step_replays"] = pcts(lper)
            log(name, legs[name])
            del lw
            torch.cuda.empty_cache()
        rec["legs"] = legs
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
