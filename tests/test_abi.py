"""The C ABI library: it loads, exports every entry point the header declares,
and rejects bad arguments on the host before anything is launched.  No kernel
runs here (CPU-only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsv4.h")


@pytest.fixture(scope="module")
def K():
    import torch  # noqa: F401  (one HIP runtime for torch and the library)
    import compressed_sparse_kv_csa_amd as K
    if not os.path.exists(K.LIB_PATH):
        from compressed_sparse_kv_csa_amd import build
        build.build()
    K.lib()
    return K


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsv4_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(K):
    names = declared_symbols()
    assert len(names) >= 9
    for n in names:
        assert hasattr(K.lib(), n), n
    assert set(names) == set(K.EXPORTS)


def test_version_and_empty_error(K):
    assert K.dsv4_version().startswith("dsv4")


def _rc(v):
    return ctypes.c_int(v).value


def test_compress_rejects_bad_args(K):
    L = K.lib()
    fake = ctypes.c_void_p(0x1000)
    assert _rc(L.dsv4_compress(None, fake, 1, fake, 1, 8, 8, 4, 1, 0, 1e4, None, fake, 1, None)) == K.DSV4_EINVAL
    assert "NULL" in K.dsv4_last_error()
    assert _rc(L.dsv4_compress(fake, fake, 1, fake, 1, 8, 7, 4, 1, 0, 1e4, None, fake, 1, None)) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_compress(fake, fake, 1, fake, 1, 8, 8, 0, 1, 0, 1e4, None, fake, 1, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_compress(fake, fake, 7, fake, 1, 8, 8, 4, 1, 0, 1e4, None, fake, 1, None)) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_compress(fake, fake, 1, fake, 1, 8, 8, 4, 1, 3, 1e4, None, fake, 1, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_compress(fake, fake, 1, fake, 65536, 8, 8, 4, 1, 0, 1e4, None, fake, 1, None)) == K.DSV4_ENOTSUP


def test_rope_rejects_bad_args(K):
    L = K.lib()
    fake = ctypes.c_void_p(0x1000)
    other = ctypes.c_void_p(0x2000)
    assert _rc(L.dsv4_rope(fake, 1, other, 1, 4, 8, 16, fake, 1e4, 0, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_rope(fake, 2, other, 1, 4, 8, 4, fake, 1e4, 0, None)) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_rope(fake, 4, other, 1, 4, 8, 4, fake, 1e4, 0, None)) == K.DSV4_ENOTSUP   # F16 input
    assert _rc(L.dsv4_rope(fake, 1, other, 1, 4, 8, 4, fake, 0.0, 0, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_rope(fake, 1, fake, 4, 4, 8, 4, fake, 1e4, 0, None)) == K.DSV4_EINVAL     # in place, dtypes differ


def _queries(K, n=4):
    fake = ctypes.c_void_p(0x1000)
    return K.Queries(n, 1, fake.value, fake.value, None)


def _rows(K, dtype, dim, **kw):
    fake = 0x1000
    r = K.Rows(fake, None, None, dtype, dim, 0, 16, fake, None)
    for k, v in kw.items():
        setattr(r, k, v)
    return r


def test_index_topk_rejects_bad_args(K):
    L = K.lib()
    fake = ctypes.c_void_p(0x1000)
    q = _queries(K)
    kp = _rows(K, K.DSV4_BF16, 128)
    ws_need = L.dsv4_index_topk_workspace(4, 16, 8)
    assert ws_need > 0
    args = lambda **o: [ctypes.byref(o.get("q", q)), fake, None, o.get("qdt", K.DSV4_BF16), fake, o.get("H", 64),
                        o.get("Di", 128), ctypes.byref(o.get("kp", kp)), 4, o.get("k", 8), o.get("sc", 0.1), fake,
                        None, o.get("ws", fake), o.get("wsb", ws_need), None]
    assert _rc(L.dsv4_index_topk(*args(k=0))) == K.DSV4_EINVAL
    assert _rc(L.dsv4_index_topk(*args(k=4096))) == K.DSV4_EINVAL
    assert _rc(L.dsv4_index_topk(*args(H=8))) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_index_topk(*args(Di=100, kp=_rows(K, K.DSV4_BF16, 100)))) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_index_topk(*args(kp=_rows(K, K.DSV4_F32, 128)))) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_index_topk(*args(sc=-1.0))) == K.DSV4_EINVAL
    assert _rc(L.dsv4_index_topk(*args(ws=None))) == K.DSV4_EWORKSPACE
    assert _rc(L.dsv4_index_topk(*args(wsb=ws_need - 1))) == K.DSV4_EWORKSPACE
    assert _rc(L.dsv4_index_topk(*args(qdt=K.DSV4_MXFP4, kp=_rows(K, K.DSV4_MXFP4, 128)))) == K.DSV4_EINVAL
    bad_q = K.Queries(4, 0, fake.value, fake.value, None)
    assert _rc(L.dsv4_index_topk(*args(q=bad_q))) == K.DSV4_EINVAL
    for stride in (1 << 29, 65535 * 1024 + 1):   # more than 65535 * 1024 entries per sequence
        huge = _rows(K, K.DSV4_BF16, 128, seq_stride=stride)
        assert _rc(L.dsv4_index_topk(*args(kp=huge, k=2048, ws=fake, wsb=1 << 62))) == K.DSV4_ENOTSUP


def test_attention_rejects_bad_args(K):
    L = K.lib()
    fake = ctypes.c_void_p(0x1000)
    q = _queries(K)
    win = _rows(K, K.DSV4_BF16, 512, first_tok=0x1000)
    pool = _rows(K, K.DSV4_BF16, 512)
    base = dict(qdt=K.DSV4_BF16, H=64, D=512, W=128, k=16, win=win, pool=pool, R=64, odt=K.DSV4_BF16)

    def call(**o):
        a = dict(base, **o)
        return _rc(L.dsv4_sparse_attn(ctypes.byref(q), fake, a["qdt"], a["H"], a["D"], ctypes.byref(a["win"]),
                                      a["W"], ctypes.byref(a["pool"]), fake, a["k"], None, 0.04, a["R"], 1.6e5,
                                      fake, a["odt"], fake, 1 << 40, None))
    assert call(D=256, win=_rows(K, K.DSV4_BF16, 256, first_tok=0x1000), pool=_rows(K, K.DSV4_BF16, 256)) == K.DSV4_ENOTSUP
    assert call(D=256) == K.DSV4_EINVAL                              # rows of another dim
    assert call(H=8) == K.DSV4_ENOTSUP
    assert call(k=4096) == K.DSV4_EINVAL
    assert call(R=65) == K.DSV4_EINVAL
    assert call(odt=3) == K.DSV4_ENOTSUP
    assert call(win=_rows(K, K.DSV4_BF16, 512)) == K.DSV4_EINVAL     # window without first_tok
    assert call(pool=_rows(K, K.DSV4_FP8R, 512, tail=64)) == K.DSV4_EINVAL   # FP8R without row_scale
    assert call(qdt=K.DSV4_F32) == K.DSV4_ENOTSUP                    # fp32 queries, bf16 rows
    assert _rc(L.dsv4_hca_attn(ctypes.byref(q), fake, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128,
                               ctypes.byref(pool), 0, None, 0.04, 64, 1.6e5, fake, K.DSV4_BF16, fake, 1 << 40,
                               None)) == K.DSV4_EINVAL


def test_workspace_sizes(K):
    L = K.lib()
    assert L.dsv4_attn_workspace(8192, 64, 512, 640) == 0          # prefill: no split partials
    assert L.dsv4_attn_workspace(0, 64, 512, 640) == 0             # no query rows
    assert L.dsv4_attn_workspace(8, 64, 512, 8320) > 8 * 64 * 512 * 4
    assert L.dsv4_index_topk_workspace(8, 262144, 1024) >= 8 * 262144 * 4


def test_batch_invariant_switch(K):
    """The mode switch returns the previous setting; in batch-invariant mode a
    short decode batch needs no split workspace (one workgroup per query)."""
    L = K.lib()
    prev = K.dsv4_set_batch_invariant(True)
    try:
        assert K.dsv4_set_batch_invariant(True) is True
        assert L.dsv4_attn_workspace(32, 64, 512, 640) == 0
        assert K.dsv4_set_batch_invariant(False) is True
        assert L.dsv4_attn_workspace(32, 64, 512, 640) > 0
    finally:
        K.dsv4_set_batch_invariant(prev)


def test_diagnostics_switch(K):
    """The diagnostics switch returns the previous setting; reading the counters
    into a NULL buffer is rejected before any device call."""
    prev = K.dsv4_set_diagnostics(True)
    try:
        assert K.dsv4_set_diagnostics(False) is True
        assert K.dsv4_set_diagnostics(False) is False
        assert K.lib().dsv4_read_diagnostics(None, 0) == K.DSV4_EINVAL
        assert "NULL" in K.dsv4_last_error()
    finally:
        K.dsv4_set_diagnostics(prev)


def test_quantize_rejects_bad_args(K):
    L = K.lib()
    fake = ctypes.c_void_p(0x1000)
    assert _rc(L.dsv4_quantize(fake, 0, 4, 512, 64, fake, fake, None, K.DSV4_BF16, None)) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_quantize(fake, 0, 4, 500, 64, fake, fake, None, K.DSV4_FP8R, None)) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_quantize(fake, 0, 4, 512, 63, fake, fake, None, K.DSV4_FP8R, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_quantize(fake, 0, 4, 512, 0, fake, None, None, K.DSV4_FP8R, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_quantize(fake, 0, 4, 128, 32, fake, None, fake, K.DSV4_MXFP4, None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_quantize(fake, 9, 4, 128, 0, fake, None, fake, K.DSV4_MXFP4, None)) == K.DSV4_ENOTSUP
    assert _rc(L.dsv4_quantize(None, 0, 0, 128, 0, None, None, None, K.DSV4_MXFP4, None)) == K.DSV4_OK


def _cache(K, **over):
    """A well-formed CSA cache descriptor on fake device addresses (never
    dereferenced: every case below fails validation or appends 0 tokens)."""
    f = 0x1000
    st = dict(dim=512, rope_dim=64, pos_bias=f, buf=f, pool=f, row_scale=f, blk_scale=None,
              pool_dtype=K.DSV4_FP8R, tail=64, pool_cap=64, count=f)
    ix = dict(dim=128, rope_dim=0, pos_bias=f, buf=f, pool=f, row_scale=None, blk_scale=f,
              pool_dtype=K.DSV4_MXFP4, tail=0, pool_cap=64, count=f)
    st.update(over.pop("kv", {}))
    ix.update(over.pop("idx", {}))
    c = dict(n_seq=2, m=4, overlap=1, rope_theta=1.6e5, pos0=None, len=f, win=f, win_scale=f,
             win_dtype=K.DSV4_FP8R, win_tail=64, win_cap=128, win_dim=512, win_rope_dim=64, win_count=f,
             win_first=f)
    c.update(over)
    return K.Cache(kv=K.Stream(**st), idx=K.Stream(**ix), **c)


def test_cache_append_rejects_bad_args(K):
    L = K.lib()
    f = ctypes.c_void_p(0x1000)

    def call(cache, n=1, kv=f, idx=f, dt=K.DSV4_BF16):
        return _rc(L.dsv4_cache_append(ctypes.byref(cache), n, None, kv, f, f, idx, idx, dt, None))

    assert _rc(L.dsv4_cache_append(None, 1, None, f, f, f, f, f, K.DSV4_BF16, None)) == K.DSV4_EINVAL
    assert call(_cache(K), n=0) == K.DSV4_OK                      # nothing to append: nothing launched
    assert call(_cache(K), n=-1) == K.DSV4_EINVAL
    assert call(_cache(K, n_seq=0)) == K.DSV4_EINVAL
    assert call(_cache(K, m=0)) == K.DSV4_ENOTSUP
    assert call(_cache(K, len=None)) == K.DSV4_EINVAL
    assert call(_cache(K), dt=K.DSV4_FP8R) == K.DSV4_ENOTSUP     # inputs are f32 or bf16
    assert call(_cache(K, kv=dict(dim=500))) == K.DSV4_ENOTSUP
    assert call(_cache(K, kv=dict(row_scale=None))) == K.DSV4_EINVAL
    assert call(_cache(K, kv=dict(tail=60))) == K.DSV4_ENOTSUP
    assert call(_cache(K, kv=dict(buf=None))) == K.DSV4_EINVAL
    assert call(_cache(K, kv=dict(rope_dim=66))) == K.DSV4_EINVAL
    assert call(_cache(K, idx=dict(blk_scale=None))) == K.DSV4_EINVAL
    assert call(_cache(K, idx=dict(tail=8))) == K.DSV4_EINVAL
    assert call(_cache(K), idx=None) == K.DSV4_EINVAL             # the idx stream needs its inputs
    assert call(_cache(K, win_dtype=K.DSV4_MXFP4, win_tail=0)) == K.DSV4_ENOTSUP
    assert call(_cache(K, win_dim=256)) == K.DSV4_EINVAL
    assert call(_cache(K), kv=None) == K.DSV4_EINVAL
    assert call(_cache(K, win_cap=-1)) == K.DSV4_EINVAL
    assert call(_cache(K, rope_theta=0.0)) == K.DSV4_EINVAL
    assert "rope_theta" in K.dsv4_last_error()


def test_ring_windows_only(K):
    """The ring layout is a window layout: a pool (no first_tok) cannot be one."""
    L = K.lib()
    f = ctypes.c_void_p(0x1000)
    q = K.Queries(1, 1, 0x1000, 0x1000, None)
    pool = K.Rows(0x1000, None, None, K.DSV4_BF16, 512, 0, 16, 0x1000, None, 1)
    rc = _rc(L.dsv4_sparse_attn(ctypes.byref(q), f, K.DSV4_BF16, 64, 512, None, 0, ctypes.byref(pool), f, 8,
                                None, 0.04, 64, 1e4, f, K.DSV4_BF16, f, 1 << 30, None))
    assert rc == K.DSV4_EINVAL and "ring" in K.dsv4_last_error()
    kp = K.Rows(0x1000, None, None, K.DSV4_BF16, 128, 0, 16, 0x1000, None, 1)
    rc = _rc(L.dsv4_index_topk(ctypes.byref(q), f, None, K.DSV4_BF16, f, 64, 128, ctypes.byref(kp), 4, 8, 1.0,
                               f, None, f, 1 << 30, None))
    assert rc == K.DSV4_EINVAL and "ring" in K.dsv4_last_error()
    win = K.Rows(0x1000, None, None, K.DSV4_BF16, 512, 0, 0, 0x1000, 0x1000, 1)   # ring of stride 0
    rc = _rc(L.dsv4_sparse_attn(ctypes.byref(q), f, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128, None, None, 0,
                                None, 0.04, 64, 1e4, f, K.DSV4_BF16, f, 1 << 30, None))
    assert rc == K.DSV4_EINVAL


def test_linear_rejects_bad_args(K):
    L = K.lib()
    f = ctypes.c_void_p(0x1000)

    def call(M=4, N=4, Kd=64, ldx=64, ldw=64, ldy=4, dt=0, groups=1, gx=0, gw=0, gy=0, x=f):
        return _rc(L.dsv4_linear(x, ldx, f, ldw, f, ldy, dt, M, N, Kd, groups, gx, gw, gy, None))

    assert call(M=0) == K.DSV4_OK                     # empty product: nothing launched
    assert call(M=-1) == K.DSV4_EINVAL
    assert call(x=None) == K.DSV4_EINVAL
    assert call(Kd=96, ldx=96, ldw=96) == K.DSV4_ENOTSUP   # K not a multiple of 64
    assert call(dt=K.DSV4_FP8R) == K.DSV4_ENOTSUP
    assert call(ldx=32) == K.DSV4_EINVAL              # row stride below K
    assert call(ldy=2) == K.DSV4_EINVAL
    assert call(ldx=68) == K.DSV4_EINVAL              # rows not 16-byte aligned
    assert call(groups=2, gx=4) == K.DSV4_EINVAL


def test_index_topk_noalloc_rejects_bad_args(K):
    """The allocation-free variant checks its arguments like dsv4_index_topk and
    refuses, before touching the device, a call whose scratch need exceeds the
    static array."""
    L = K.lib()
    fake = ctypes.c_void_p(0x1000)
    q = _queries(K)
    args = lambda **o: [ctypes.byref(o.get("q", q)), fake, None, K.DSV4_BF16, fake, 64, 128,
                        ctypes.byref(o.get("kp", _rows(K, K.DSV4_BF16, 128))), 4, o.get("k", 8), 0.1, fake, None, None]
    assert _rc(L.dsv4_index_topk_noalloc(*args(k=0))) == K.DSV4_EINVAL
    big = _rows(K, K.DSV4_BF16, 128, seq_stride=1 << 21)   # 4 rows x 2^21 entries x 4 B = 32 MiB of scores
    assert L.dsv4_index_topk_workspace(4, 1 << 21, 8) > K.NOALLOC_SCRATCH_BYTES
    assert _rc(L.dsv4_index_topk_noalloc(*args(kp=big))) == K.DSV4_EWORKSPACE
    assert "scratch" in K.dsv4_last_error()


def test_empty_calls_queue_nothing(K):
    """A call with nothing to do returns DSV4_OK and accepts NULL data
    pointers (no kernel is launched, so this runs without a GPU)."""
    L = K.lib()
    empty_q = K.Queries(0, 1, None, None, None)
    win = _rows(K, K.DSV4_BF16, 512, first_tok=0x1000)
    pool = _rows(K, K.DSV4_BF16, 512)
    assert _rc(L.dsv4_sparse_attn(ctypes.byref(empty_q), None, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128,
                                  ctypes.byref(pool), None, 0, None, 0.04, 64, 1.6e5, None, K.DSV4_BF16, None, 0,
                                  None)) == K.DSV4_OK
    assert _rc(L.dsv4_sparse_attn(ctypes.byref(empty_q), None, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128,
                                  ctypes.byref(pool), None, 512, None, 0.04, 64, 1.6e5, None, K.DSV4_BF16, None, 0,
                                  None)) == K.DSV4_OK   # picks expected, no idx: nothing to pick for
    assert _rc(L.dsv4_hca_attn(ctypes.byref(empty_q), None, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128,
                               ctypes.byref(pool), 128, None, 0.04, 64, 1.6e5, None, K.DSV4_BF16, None, 0,
                               None)) == K.DSV4_OK
    assert _rc(L.dsv4_rope(None, K.DSV4_BF16, None, K.DSV4_BF16, 0, 512, 64, None, 1.6e5, 0, None)) == K.DSV4_OK
    assert _rc(L.dsv4_compress(None, None, K.DSV4_BF16, None, 1, 3, 512, 4, 1, 64, 1.6e5, None, None,
                               K.DSV4_BF16, None)) == K.DSV4_OK   # seq_len < m: no entry
    kp = _rows(K, K.DSV4_BF16, 128)
    assert _rc(L.dsv4_index_topk(ctypes.byref(empty_q), None, None, K.DSV4_BF16, None, 64, 128, ctypes.byref(kp),
                                 4, 512, 0.01, None, None, None, 0, None)) == K.DSV4_OK
    # with rows to do, the same NULL pointers are errors
    one_q = K.Queries(1, 1, 0x1000, 0x1000, None)
    assert _rc(L.dsv4_sparse_attn(ctypes.byref(one_q), None, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128,
                                  ctypes.byref(pool), None, 0, None, 0.04, 64, 1.6e5, None, K.DSV4_BF16, None, 0,
                                  None)) == K.DSV4_EINVAL
    assert _rc(L.dsv4_sparse_attn(ctypes.byref(one_q), 0x1000, K.DSV4_BF16, 64, 512, ctypes.byref(win), 128,
                                  ctypes.byref(pool), None, 512, None, 0.04, 64, 1.6e5, 0x1000, K.DSV4_BF16, None, 0,
                                  None)) == K.DSV4_EINVAL   # picks expected, idx NULL
    assert _rc(L.dsv4_rope(None, K.DSV4_BF16, None, K.DSV4_BF16, 4, 512, 64, None, 1.6e5, 0, None)) == K.DSV4_EINVAL
