"""The C ABI library loads, exports every symbol include/wushkv.h declares, and
rejects bad arguments on the host with the documented status codes before
anything is launched.  No GPU needed: every call here fails validation (fake
pointers are never dereferenced), or only computes sizes."""
import ctypes
import os
import re
import subprocess

import pytest

import bit_kv_cache_amd as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wushkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(W.LIB_PATH):
        pytest.skip("libwushkv.so not built (run __graft_entry__.build())")
    return W.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wushkv_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert set(names) == set(W.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", W.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (wushkv_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings_and_version(lib):
    assert W.status_string(0) == "ok"
    assert "capacity" in W.status_string(W.ERR_CAPACITY)
    assert W.status_string(99) == "unknown status"
    assert lib.wushkv_abi_version() == 5


def _spec(**kw):
    base = dict(batch=2, num_kv_heads=8, head_dim=128, capacity=8256, sink=64, recent=256, chunk=8,
                bits_k=2, bits_v=3, quant_k=W.Q_AFFINE, quant_v=W.Q_QUEST)
    base.update(kw)
    return W.CacheSpec(**base)


def test_plane_bytes_follow_the_layout(lib):
    s = _spec()
    pb = s.plane_bytes()
    heads = 2 * 8
    body_cap = -(-(8256 - 64) // 64) * 64
    assert pb["sink_k"] == heads * 64 * 128 * 2
    assert pb["ring_v"] == heads * (256 + 8) * 128 * 2
    assert pb["codes_k"] == heads * body_cap * 128 * 2 // 8
    assert pb["codes_v"] == heads * (body_cap // 64) * 64 * 128 * 3 // 8
    assert pb["par_k"] == heads * body_cap * 2 * 2
    assert pb["par_v"] == heads * body_cap * 1 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), W.ERR_SHAPE),
    (dict(bits_k=5), W.ERR_SHAPE),
    (dict(bits_v=1), W.ERR_SHAPE),
    (dict(chunk=0), W.ERR_SHAPE),
    (dict(recent=250), W.ERR_SHAPE),          # recent must be a multiple of chunk
    (dict(quant_k=7), W.ERR_SHAPE),
    (dict(pct_lo=60.0, pct_hi=40.0), W.ERR_SHAPE),
    (dict(pct_lo=10.0), W.ERR_UNSUPPORTED),    # needs 14 order statistics from the bottom
    (dict(clip_mult=0.0, quant_v=W.Q_QUEST), W.ERR_SHAPE),
    (dict(batch=0), W.ERR_SHAPE),
    (dict(), W.OK),
])
def test_descriptor_checks(lib, kw, status):
    d = _spec(**kw).desc()
    assert lib.wushkv_cache_check(ctypes.byref(d)) == status


def _fake_planes(d, align=16):
    for i, p in enumerate(W.PLANES):
        setattr(d, p, 0x10000 * (i + 1) + (0 if align == 16 else 4))


def test_append_flush_validation(lib):
    d = _spec().desc()
    f = lib.wushkv_append_flush
    kv = ctypes.c_void_p(0x900000)
    # null planes
    assert f(ctypes.byref(d), 0, 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    _fake_planes(d)
    assert f(ctypes.byref(d), 0, 1, None, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    assert f(ctypes.byref(d), 0, 1, kv, kv, 9, kv, None) == W.ERR_SHAPE
    assert f(ctypes.byref(d), -1, 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_SHAPE
    assert f(ctypes.byref(d), 8000, 257, kv, kv, W.DT_BF16, kv, None) == W.ERR_CAPACITY
    assert f(ctypes.byref(d), 0, 1, ctypes.c_void_p(0x900004), kv, W.DT_BF16, kv, None) == W.ERR_ALIGN
    assert f(ctypes.byref(d), 5, 0, None, None, W.DT_BF16, None, None) == W.OK  # no-op
    _fake_planes(d, align=4)
    assert f(ctypes.byref(d), 0, 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_ALIGN


def test_query_transform_validation(lib):
    f = lib.wushkv_query_transform
    p = ctypes.c_void_p(0x900000)
    assert f(p, p, W.DT_BF16, 1, 30, 8, 128, p, None) == W.ERR_SHAPE   # 30 % 8 != 0
    assert f(p, p, W.DT_BF16, 1, 32, 8, 80, p, None) == W.ERR_SHAPE
    assert f(None, p, W.DT_BF16, 1, 32, 8, 128, p, None) == W.ERR_NULL
    assert f(p, ctypes.c_void_p(0x900002), W.DT_BF16, 1, 32, 8, 128, p, None) == W.ERR_ALIGN


def test_decode_validation_and_workspace(lib):
    d = _spec().desc()
    _fake_planes(d)
    f = lib.wushkv_decode_attention
    p = ctypes.c_void_p(0x900000)
    ws_need = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    P = lib.wushkv_decode_num_splits(ctypes.byref(d), 8000, 32, 0)
    assert P >= 1
    rows = 2 * 32 * (P + 1)
    assert ws_need >= rows * 128 * 4 + rows * 8
    assert lib.wushkv_decode_num_splits(ctypes.byref(d), 8000, 32, 7) == 7
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, 32, 0, p, ws_need - 1, p, None) == W.ERR_WORKSPACE
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, 32, 0, None, ws_need, p, None) == W.ERR_WORKSPACE
    assert f(ctypes.byref(d), 9000, p, W.DT_BF16, p, 32, 0, p, ws_need, p, None) == W.ERR_CAPACITY
    assert f(ctypes.byref(d), 0, p, W.DT_BF16, p, 32, 0, p, ws_need, p, None) == W.ERR_SHAPE
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, 30, 0, p, ws_need, p, None) == W.ERR_SHAPE
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, 8 * 17, 0, p, ws_need, p, None) == W.ERR_SHAPE  # G = 17
    assert f(ctypes.byref(d), 8000, None, W.DT_BF16, p, 32, 0, p, ws_need, p, None) == W.ERR_NULL
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, 32, -1, p, ws_need, p, None) == W.ERR_SHAPE
    assert lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 0, 32, 0) == 0


def test_fused_decode_validation(lib):
    """The fused entry checks its arguments like the plain decode (nothing launches)."""
    d = _spec().desc()
    _fake_planes(d)
    f = lib.wushkv_decode_attention_fused
    p = ctypes.c_void_p(0x900000)
    ws_need = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, None, p, 32, 0, p, ws_need, p, None) == W.ERR_NULL
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, ctypes.c_void_p(0x900004), p, 32, 0, p, ws_need, p,
             None) == W.ERR_ALIGN
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, None, 32, 0, p, ws_need, p, None) == W.ERR_NULL
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, p, 32, 0, p, ws_need - 1, p, None) == W.ERR_WORKSPACE
    assert f(ctypes.byref(d), 9000, p, W.DT_BF16, p, p, 32, 0, p, ws_need, p, None) == W.ERR_CAPACITY
    assert f(ctypes.byref(d), 8000, p, W.DT_BF16, p, p, 30, 0, p, ws_need, p, None) == W.ERR_SHAPE


def test_product_package_does_not_use_the_oracle():
    pkg = os.path.join(ROOT, "bit_kv_cache_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.replace("oracle of", ""), fn


def test_calib_validation_and_workspace(lib):
    """Calibration sums: argument checks on the host (nothing launches) and the
    workspace size (10 upper-triangle 32 x 32 fp32 tiles per partial)."""
    f = lib.wushkv_calib_stats
    wsb = lib.wushkv_calib_workspace_bytes
    p = ctypes.c_void_p(0x900000)
    need = wsb(128, 32, 1024, 128, 4)
    assert need > 0 and need % (10 * 1024 * 4) == 0
    assert (need // (10 * 1024 * 4)) % 8 == 0          # a whole number of partials per group
    assert wsb(128, 32, 1024, 64, 4) == 0 and wsb(128, 30, 1024, 128, 4) == 0 and wsb(0, 8, 1, 128, 1) == 0
    n1 = wsb(2, 8, 64, 128, 1)
    assert f(p, W.DT_BF16, 2, 8, 64, 128, 3, p, n1, p, None) == W.ERR_SHAPE       # 8 % 3
    assert f(p, W.DT_BF16, 0, 8, 64, 128, 1, p, n1, p, None) == W.ERR_SHAPE
    assert f(p, W.DT_BF16, 2, 8, 0, 128, 1, p, n1, p, None) == W.ERR_SHAPE
    assert f(p, 9, 2, 8, 64, 128, 1, p, n1, p, None) == W.ERR_SHAPE
    assert f(p, W.DT_F32, 2, 8, 64, 128, 1, p, n1, p, None) == W.ERR_UNSUPPORTED
    assert f(p, W.DT_BF16, 2, 8, 64, 64, 1, p, n1, p, None) == W.ERR_UNSUPPORTED
    assert f(None, W.DT_BF16, 2, 8, 64, 128, 1, p, n1, p, None) == W.ERR_NULL
    assert f(p, W.DT_BF16, 2, 8, 64, 128, 1, p, n1, None, None) == W.ERR_NULL
    assert f(ctypes.c_void_p(0x900002), W.DT_BF16, 2, 8, 64, 128, 1, p, n1, p, None) == W.ERR_ALIGN
    assert f(p, W.DT_BF16, 2, 8, 64, 128, 1, p, n1 - 1, p, None) == W.ERR_WORKSPACE
    assert f(p, W.DT_BF16, 2, 8, 64, 128, 1, None, n1, p, None) == W.ERR_WORKSPACE


def test_ragged_validation(lib):
    """Ragged append and decode check every sequence's count on the host."""
    d = _spec(batch=3).desc()
    _fake_planes(d)
    kv = ctypes.c_void_p(0x900000)
    arr = lambda *v: (ctypes.c_int64 * len(v))(*v)
    fa = lib.wushkv_append_flush_ragged
    assert fa(ctypes.byref(d), None, 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    assert fa(ctypes.byref(d), arr(0, -1, 5), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_SHAPE
    assert fa(ctypes.byref(d), arr(0, 8256, 5), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_CAPACITY
    assert fa(ctypes.byref(d), arr(0, 3, 5), 0, kv, kv, W.DT_BF16, kv, None) == W.OK   # no-op
    big = _spec(batch=300).desc()
    _fake_planes(big)
    assert fa(ctypes.byref(big), (ctypes.c_int64 * 300)(), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_UNSUPPORTED
    fd = lib.wushkv_decode_attention_ragged
    p = ctypes.c_void_p(0x900000)
    ws = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    assert fd(ctypes.byref(d), None, p, W.DT_BF16, None, p, 32, 0, p, ws, p, None) == W.ERR_NULL
    assert fd(ctypes.byref(d), arr(5, 0, 7), p, W.DT_BF16, None, p, 32, 0, p, ws, p, None) == W.ERR_SHAPE
    assert fd(ctypes.byref(d), arr(5, 9000, 7), p, W.DT_BF16, None, p, 32, 0, p, ws, p, None) == W.ERR_CAPACITY
    assert fd(ctypes.byref(d), arr(5, 8000, 7), p, W.DT_BF16, None, p, 32, 0, p, ws - 1, p, None) == W.ERR_WORKSPACE


def test_device_count_validation(lib):
    """Device-count append and decode: host-side checks only (the counts themselves
    are read, and range-checked, by the kernels)."""
    d = _spec(batch=3).desc()
    _fake_planes(d)
    kv = ctypes.c_void_p(0x900000)
    fa = lib.wushkv_append_flush_device
    assert fa(ctypes.byref(d), None, 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    assert fa(ctypes.byref(d), ctypes.c_void_p(0x900002), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_ALIGN
    assert fa(ctypes.byref(d), kv, -1, kv, kv, W.DT_BF16, kv, None) == W.ERR_SHAPE
    assert fa(ctypes.byref(d), kv, 8257, kv, kv, W.DT_BF16, kv, None) == W.ERR_CAPACITY
    assert fa(ctypes.byref(d), kv, 0, kv, kv, W.DT_BF16, kv, None) == W.OK        # no-op: counts unchanged
    assert fa(ctypes.byref(d), kv, 1, None, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    fd = lib.wushkv_decode_attention_device
    p = ctypes.c_void_p(0x900000)
    ws = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    assert fd(ctypes.byref(d), None, 8000, p, W.DT_BF16, None, p, 32, 0, p, ws, p, None) == W.ERR_NULL
    assert fd(ctypes.byref(d), ctypes.c_void_p(0x900001), 8000, p, W.DT_BF16, None, p, 32, 0, p, ws, p,
              None) == W.ERR_ALIGN
    assert fd(ctypes.byref(d), p, 0, p, W.DT_BF16, None, p, 32, 0, p, ws, p, None) == W.ERR_SHAPE
    assert fd(ctypes.byref(d), p, 9000, p, W.DT_BF16, None, p, 32, 0, p, ws, p, None) == W.ERR_CAPACITY
    assert fd(ctypes.byref(d), p, 8000, p, W.DT_BF16, None, p, 32, 0, p, ws - 1, p, None) == W.ERR_WORKSPACE
    big = _spec(batch=300).desc()      # no per-sequence array in the launch: any batch size
    _fake_planes(big)
    assert fa(ctypes.byref(big), kv, 0, kv, kv, W.DT_BF16, kv, None) == W.OK


def test_paged_validation_and_pool_bytes(lib):
    """Page-table checks on the host and pool sizes (no launches)."""
    s = _spec(batch=3)
    d = s.desc()
    _fake_planes(d)
    kv = ctypes.c_void_p(0x900000)
    arr = lambda *v: (ctypes.c_int64 * len(v))(*v)
    body = -(-(8256 - 64) // 64) * 64                       # body rows of a full sequence
    pages = lambda tab=0x800000, pt=256, mp=-(-body // 256), npg=40: W.PagesDesc(tab, pt, mp, npg)
    fa, fd = lib.wushkv_append_flush_paged, lib.wushkv_decode_attention_paged
    ok = pages()
    assert fa(ctypes.byref(d), None, arr(0, 0, 0), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    assert fa(ctypes.byref(d), ctypes.byref(pages(tab=0)), arr(0, 0, 0), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_NULL
    assert fa(ctypes.byref(d), ctypes.byref(pages(tab=0x800002)), arr(0, 0, 0), 1, kv, kv, W.DT_BF16, kv,
              None) == W.ERR_ALIGN
    assert fa(ctypes.byref(d), ctypes.byref(pages(pt=100)), arr(0, 0, 0), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_SHAPE
    assert fa(ctypes.byref(d), ctypes.byref(pages(npg=0)), arr(0, 0, 0), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_SHAPE
    assert fa(ctypes.byref(d), ctypes.byref(pages(mp=2)), arr(0, 0, 0), 1, kv, kv, W.DT_BF16, kv,
              None) == W.ERR_CAPACITY
    assert fa(ctypes.byref(d), ctypes.byref(ok), arr(0, 3, 5), 0, kv, kv, W.DT_BF16, kv, None) == W.OK   # no-op
    assert fa(ctypes.byref(d), ctypes.byref(ok), arr(0, 8256, 5), 1, kv, kv, W.DT_BF16, kv, None) == W.ERR_CAPACITY
    ws = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    assert fd(ctypes.byref(d), ctypes.byref(pages(pt=64 * 3 + 1)), arr(5, 6, 7), kv, W.DT_BF16, None, kv, 32, 0, kv,
              ws, kv, None) == W.ERR_SHAPE
    assert fd(ctypes.byref(d), None, arr(5, 6, 7), kv, W.DT_BF16, None, kv, 32, 0, kv, ws, kv, None) == W.ERR_NULL
    assert fd(ctypes.byref(d), ctypes.byref(ok), arr(5, 0, 7), kv, W.DT_BF16, None, kv, 32, 0, kv, ws, kv,
              None) == W.ERR_SHAPE
    # pools: num_pages x Hkv x page_tokens rows; windows as in the unpaged cache
    pool = lambda plane: lib.wushkv_pool_bytes(ctypes.byref(d), ctypes.byref(ok), plane)
    rows = 40 * 8 * 256
    assert pool(4) == rows * 128 * 2 // 8          # codes_k, 2-bit
    assert pool(5) == rows // 64 * 64 * 128 * 3 // 8   # codes_v, 3-bit sets
    assert pool(6) == rows * 4 and pool(7) == rows * 2   # affine (s, z) keys, QuEST values
    assert pool(0) == lib.wushkv_plane_bytes(ctypes.byref(d), 0)
    assert lib.wushkv_pool_bytes(ctypes.byref(d), ctypes.byref(pages(pt=100)), 4) == 0


def test_decode_step_validation(lib):
    """Every check of the fused step runs before anything is enqueued."""
    d = _spec(batch=2).desc()
    _fake_planes(d)
    p = ctypes.c_void_p(0x900000)
    ws = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    f = lambda nb, kn=p, tinv=p, wsb=ws, q=p: lib.wushkv_decode_step(
        ctypes.byref(d), nb, kn, p, W.DT_BF16, p, q, W.DT_BF16, tinv, p, 32, 0, p, wsb, p, None)
    assert f(10, tinv=None) == W.ERR_NULL
    assert f(10, kn=None) == W.ERR_NULL
    assert f(-1) == W.ERR_SHAPE
    assert f(8256) == W.ERR_CAPACITY
    assert f(7999, wsb=ws - 1) == W.ERR_WORKSPACE
    assert f(10, kn=ctypes.c_void_p(0x900004)) == W.ERR_ALIGN
    assert f(10, q=ctypes.c_void_p(0x900008)) == W.ERR_ALIGN


def test_device_step_validation(lib):
    d = _spec(batch=3).desc()
    _fake_planes(d)
    p = ctypes.c_void_p(0x900000)
    ws = lib.wushkv_decode_workspace_bytes(ctypes.byref(d), 8000, 32, 0)
    f = lambda cnt=p, mt=8000, wsb=ws, tinv=p: lib.wushkv_decode_step_device(
        ctypes.byref(d), cnt, mt, p, p, W.DT_BF16, p, p, W.DT_BF16, tinv, p, 32, 0, p, wsb, p, None)
    assert f(cnt=None) == W.ERR_NULL
    assert f(tinv=None) == W.ERR_NULL
    assert f(cnt=ctypes.c_void_p(0x900002)) == W.ERR_ALIGN
    assert f(mt=0) == W.ERR_SHAPE
    assert f(mt=9000) == W.ERR_CAPACITY
    assert f(wsb=ws - 1) == W.ERR_WORKSPACE


def test_hadamard_flush_argument_checks(lib):
    """wushkv_append_flush_hadamard: the scale must be a nonzero, finite fp16 value; the
    usual pointer checks; nothing is launched on these failures."""
    s = _spec(quant_k=W.Q_QUEST)
    import ctypes as C
    desc = s.desc()
    for p in W.PLANES:
        setattr(desc, p, 256)
    fake = C.c_void_p(4096)
    for scale in (0.0, float("nan"), float("inf"), 0.1, 1e-9):
        assert lib.wushkv_append_flush_hadamard(C.byref(desc), 0, 16, fake, fake, W.DT_BF16, scale, None) == W.ERR_SHAPE
    ok_scale = 0.08837890625                      # fp16(1/sqrt(128))
    assert lib.wushkv_append_flush_hadamard(C.byref(desc), 0, 16, None, fake, W.DT_BF16, ok_scale, None) == W.ERR_NULL
    assert lib.wushkv_append_flush_hadamard(C.byref(desc), 0, 16, C.c_void_p(4100), fake, W.DT_BF16, ok_scale,
                                            None) == W.ERR_ALIGN
    assert lib.wushkv_append_flush_hadamard(C.byref(desc), 9000, 16, fake, fake, W.DT_BF16, ok_scale,
                                            None) == W.ERR_CAPACITY
