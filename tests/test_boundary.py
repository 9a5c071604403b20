"""The C-ABI boundary on the host: libhq.so loads and exports every function
include/hq.h declares; hq_plan's validation and sizes; argument checks that
return before any device work (no GPU is touched: every call here fails its
checks first or is host-only)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hq.h")
LIB = os.path.join(ROOT, "kv_cache_tile_amd", "libhq.so")

OK, EINVAL, ENOSPC = 0, -1, -3
F32, BF16 = 0, 1
E8, Z, A2, D4 = 8, 1, 2, 4


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from kv_cache_tile_amd import build as b
        b.build()
    L = ctypes.CDLL(LIB)
    u32, u64, f32, vp = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p
    P = ctypes.POINTER
    L.hq_plan.argtypes = [u32, u64, u64, u32, u32, f32, u32, P(u64), P(u64), P(u64), P(u64), P(u32), P(f32)]
    L.hq_encode.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, vp, u64, vp, vp, vp, vp, vp, u64, vp]
    L.hq_decode.argtypes = [vp, u64, vp, vp, vp, u32, u64, u64, u32, u32, f32, u64, vp, vp, vp]
    L.hq_kv_encode.argtypes = [vp, u32, u64, u32, u32, f32, u64, vp, u64, vp, vp, vp, vp, vp, u64, vp]
    L.hq_kv_decode.argtypes = [vp, u64, vp, vp, vp, u32, u64, u32, u32, f32, u64, vp, vp, vp]
    L.hq_strerror.argtypes = [ctypes.c_int]
    L.hq_strerror.restype = ctypes.c_char_p
    L.hq_version.restype = u32
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"hq_plan", "hq_encode", "hq_decode", "hq_kv_encode", "hq_kv_decode"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"libhq.so does not export {n}"


def plan(lib, dtype=BF16, rows=4096, cols=16384, tile=256, lat=E8, bps=4.0, kv=0):
    T, C, cap, ws = (ctypes.c_uint64() for _ in range(4))
    bound, c = ctypes.c_uint32(), ctypes.c_float()
    rc = lib.hq_plan(dtype, rows, cols, tile, lat, bps, kv, ctypes.byref(T), ctypes.byref(C), ctypes.byref(cap),
                     ctypes.byref(ws), ctypes.byref(bound), ctypes.byref(c))
    return rc, T.value, C.value, cap.value, ws.value, bound.value, c.value


def test_plan_sizes(lib):
    rc, T, C, cap, ws, bound, c = plan(lib)
    assert rc == OK
    assert T == 4096 * 16384 // 256 and C == (T + 63) // 64
    assert ws == 8 + 8 * C                      # ticket, epoch, one look-back word per group (<= C)
    assert cap >= (T * bound + 31) // 32        # every tile at its worst case fits
    assert 256 * 4 < bound < 256 * 8            # a tile's worst case lies above the 4 bps target
    assert 0.1 < c < 1.0


@pytest.mark.parametrize("args", [
    dict(tile=100), dict(tile=32), dict(cols=1000), dict(rows=0), dict(lat=3),
    dict(bps=4.1), dict(bps=1.25), dict(bps=8.25), dict(dtype=2),
])
def test_plan_rejects(lib, args):
    assert plan(lib, **args)[0] == EINVAL


def test_plan_kv_head_dims(lib):
    for hd in (64, 128, 256):
        assert plan(lib, rows=1000, cols=hd, tile=hd, kv=1, bps=2.0)[0] == OK


def test_strerror_and_version(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.hq_strerror(code)
    assert lib.hq_strerror(12345) == b"unknown error"
    assert lib.hq_version() >> 16 >= 1


def test_calls_reject_bad_pointers_before_device_work(lib):
    # fake device addresses: every call below must fail its argument checks
    # before touching them or the (absent) GPU
    rc, T, C, cap, ws, bound, c = plan(lib, rows=64, cols=1024, tile=128)
    A = 1 << 40                                     # 16-byte aligned, never dereferenced
    good = dict(x=A, pay=A, step=A, meta=A, off=A, st=A, wsp=A)

    def enc(**kw):
        a = {**good, **kw}
        return lib.hq_encode(a["x"], BF16, 64, 1024, 128, E8, 4.0, 1, a["pay"], kw.get("cap", cap), a["step"],
                             a["meta"], a["off"], a["st"], a["wsp"], kw.get("ws", ws), None)

    def dec(**kw):
        a = {**good, **kw}
        return lib.hq_decode(a["pay"], 100, a["step"], a["meta"], a["off"], BF16, 64, 1024, 128, E8, 4.0, 1,
                             a["x"], a["st"], None)

    assert enc(x=None) == EINVAL and enc(pay=None) == EINVAL and enc(wsp=None) == EINVAL
    assert enc(x=A + 4) == EINVAL                  # input not 16-byte aligned
    assert enc(wsp=A + 4) == EINVAL                # workspace not 8-byte aligned
    assert enc(cap=cap - 1) == ENOSPC and enc(ws=ws - 8) == ENOSPC
    assert dec(pay=None) == EINVAL and dec(x=None) == EINVAL and dec(st=None) == EINVAL
    assert dec(x=A + 8) == EINVAL                  # output not 16-byte aligned
    assert dec(pay=A + 4) == EINVAL                # payload not 16-byte aligned
    assert lib.hq_kv_encode(A, BF16, 100, 96, E8, 2.0, 1, A, 1 << 20, A, A, A, A, A, 1 << 20, None) == EINVAL
    assert lib.hq_kv_decode(A, 100, A, A, A, BF16, 100, 96, E8, 2.0, 1, A, A, None) == EINVAL
