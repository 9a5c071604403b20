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
    L.hq_plan_c.argtypes = [u32, u64, u64, u32, u32, f32, u32, P(u64), P(u64), P(u64), P(u64), P(u32)]
    L.hq_encode_c.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, u64, vp, vp, vp, vp, vp, u64, vp]
    L.hq_decode_c.argtypes = [vp, u64, vp, vp, vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, vp, vp]
    L.hq_rate_bracket.argtypes = [u32, f32, P(f32), P(f32)]
    L.hq_encode_rate.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, u64, vp, vp, vp, vp, vp, u64,
                                 P(f32), P(ctypes.c_double), P(u32), vp]
    L.hq_encode_length_c.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, vp]
    L.hq_rotate.argtypes = [vp, u32, u32, vp, u32, u64, vp, u32, vp]
    L.hq_act_quant.argtypes = [vp, u32, u64, u64, u32, u64, vp, vp, vp]
    L.hq_act_quant_blocked.argtypes = [vp, u32, u64, u64, u32, u64, vp, vp, vp]
    L.hq_codes_matmul_fused.argtypes = [vp, u64, vp, vp, vp, u64, u64, u32, u32, f32, vp, vp, u64, vp, vp, vp]
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
    assert ws == 768 + 8 * C                    # event word, epoch, started bits, a look-back word per group (<= C)
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


# ---------------------------------------------------------------- closed-loop rate (host side)
def plan_c(lib, c, dtype=BF16, rows=4096, cols=16384, tile=256, lat=E8, kv=0):
    T, C, cap, ws = (ctypes.c_uint64() for _ in range(4))
    bound = ctypes.c_uint32()
    rc = lib.hq_plan_c(dtype, rows, cols, tile, lat, c, kv, ctypes.byref(T), ctypes.byref(C), ctypes.byref(cap),
                       ctypes.byref(ws), ctypes.byref(bound))
    return rc, T.value, C.value, cap.value, ws.value, bound.value


def test_plan_c_matches_the_table_plan_and_shrinks_with_c(lib):
    rc, T, C, cap, ws, bound, c = plan(lib)
    assert plan_c(lib, c) == (OK, T, C, cap, ws, bound)
    bounds = [plan_c(lib, c * f)[5] for f in (0.25, 0.5, 1.0, 2.0, 4.0)]
    assert all(a > b for a, b in zip(bounds, bounds[1:]))
    for bad in (0.0, -1.0, float("nan"), float("inf"), 1e-4):   # 1e-4: tiles could pass 8191 bits
        assert plan_c(lib, bad)[0] == EINVAL


def test_rate_bracket_matches_the_oracle(lib):
    import numpy as np

    import oracle
    lo, hi = ctypes.c_float(), ctypes.c_float()
    for name, code in (("Z", Z), ("A2", A2), ("D4", D4), ("E8", E8)):
        for R in (1.0, 2.0, 3.3, 4.0, 5.75, 7.99, 8.0):
            assert lib.hq_rate_bracket(code, R, ctypes.byref(lo), ctypes.byref(hi)) == OK
            assert (lo.value, hi.value) == oracle.rate_bracket(name, float(np.float32(R)))
    for R in (0.5, 8.5, float("nan")):
        assert lib.hq_rate_bracket(E8, R, ctypes.byref(lo), ctypes.byref(hi)) == EINVAL
    assert lib.hq_rate_bracket(3, 4.0, ctypes.byref(lo), ctypes.byref(hi)) == EINVAL


def test_rate_calls_reject_before_device_work(lib):
    A = 1 << 40
    lo, hi = ctypes.c_float(), ctypes.c_float()
    lib.hq_rate_bracket(E8, 4.0, ctypes.byref(lo), ctypes.byref(hi))
    rc, T, C, cap, ws, bound = plan_c(lib, lo.value, rows=64, cols=1024, tile=128)
    assert rc == OK
    c_out, r_out, n_out = ctypes.c_float(), ctypes.c_double(), ctypes.c_uint32()

    def rate(**kw):
        a = dict(x=A, pay=A, cap=cap, wsp=A, ws=ws, R=4.0, kv=0, cols=1024, tile=128)
        a.update(kw)
        return lib.hq_encode_rate(a["x"], BF16, 64, a["cols"], a["tile"], E8, a["R"], 1, a["kv"], a["pay"],
                                  a["cap"], A, A, A, A, a["wsp"], a["ws"], ctypes.byref(c_out), ctypes.byref(r_out),
                                  ctypes.byref(n_out), None)

    assert rate(cap=cap - 1) == ENOSPC and rate(ws=ws - 8) == ENOSPC   # sized at the bracket's low end
    assert rate(R=0.5) == EINVAL and rate(R=9.0) == EINVAL
    assert rate(kv=1) == EINVAL                                        # KV needs cols == tile
    assert rate(x=None) == EINVAL and rate(pay=None) == EINVAL and rate(wsp=None) == EINVAL
    assert rate(x=A + 8) == EINVAL and rate(wsp=A + 4) == EINVAL       # 16- and 8-byte alignment

    def length(**kw):
        a = dict(x=A, words=A, c=0.3, kv=0, cols=1024, tile=128)
        a.update(kw)
        return lib.hq_encode_length_c(a["x"], BF16, 64, a["cols"], a["tile"], E8, a["c"], 1, a["kv"], a["words"],
                                      None)

    assert length(x=None) == EINVAL and length(words=None) == EINVAL
    assert length(x=A + 8) == EINVAL and length(words=A + 4) == EINVAL
    assert length(c=0.0) == EINVAL and length(c=float("inf")) == EINVAL
    assert length(kv=1) == EINVAL and length(cols=1000) == EINVAL and length(tile=96) == EINVAL
    assert lib.hq_encode_c(A, BF16, 64, 1024, 128, E8, 0.0, 1, 0, A, cap, A, A, A, A, A, ws, None) == EINVAL
    assert lib.hq_encode_c(None, BF16, 64, 1024, 128, E8, 0.3, 1, 0, A, cap, A, A, A, A, A, ws, None) == EINVAL
    assert lib.hq_decode_c(A, 100, A, A, A, BF16, 64, 1024, 128, E8, -1.0, 1, 0, A, A, None) == EINVAL
    assert lib.hq_decode_c(A, 100, A, A, A, BF16, 64, 1024, 128, E8, 0.3, 1, 1, A, A, None) == EINVAL


def test_rotate_rejects_before_device_work(lib):
    A = 1 << 40
    assert lib.hq_rotate(A, 96, 0, A, BF16, 10, A, F32, None) == EINVAL           # d is 64 or 128
    assert lib.hq_rotate(A, 128, 2, A, BF16, 10, A, F32, None) == EINVAL
    assert lib.hq_rotate(A, 128, 0, A, 3, 10, A, F32, None) == EINVAL
    assert lib.hq_rotate(None, 128, 0, A, BF16, 10, A, F32, None) == EINVAL
    assert lib.hq_rotate(A, 128, 0, A + 8, BF16, 10, A, F32, None) == EINVAL      # x not 16-byte aligned
    assert lib.hq_rotate(A, 128, 0, A, BF16, 10, A + 4, F32, None) == EINVAL
    assert lib.hq_rotate(A, 128, 0, A, BF16, 1 << 32, A, F32, None) == EINVAL
    assert lib.hq_rotate(A, 128, 0, A, BF16, 0, A, F32, None) == OK               # nothing to do


def test_int8_calls_reject_before_device_work(lib):
    A = 1 << 40
    for fn in (lib.hq_act_quant, lib.hq_act_quant_blocked):
        assert fn(None, BF16, 4, 1024, 256, 1, A, A, None) == EINVAL
        assert fn(A, BF16, 4, 1000, 256, 1, A, A, None) == EINVAL             # cols not a multiple of n
        assert fn(A, BF16, 4, 1024, 96, 1, A, A, None) == EINVAL              # n is 64, 128 or 256
        assert fn(A, 7, 4, 1024, 256, 1, A, A, None) == EINVAL
        assert fn(A, BF16, 0, 1024, 256, 1, A, A, None) == OK                 # nothing to do
    # at most 2^32 - 1 codes: row-major, 33 activations of 2^27 columns pass
    # it; blocked, 17 activations already do (rounded up to 32)
    assert lib.hq_act_quant(A, BF16, 33, 1 << 27, 256, 1, A, A, None) == EINVAL
    assert lib.hq_act_quant_blocked(A, BF16, 17, 1 << 27, 256, 1, A, A, None) == EINVAL
    c = ctypes.c_float(0.3)

    def fused(**kw):
        a = dict(pay=A, rows=16, cols=64 * 256, tile=256, lat=E8, q=A, batch=8)
        a.update(kw)
        return lib.hq_codes_matmul_fused(a["pay"], 100, A, A, A, a["rows"], a["cols"], a["tile"], a["lat"], c,
                                         a["q"], A, a["batch"], A, A, None)
    assert fused(lat=A2) == EINVAL                                                # integer codes only
    assert fused(cols=32 * 256) == EINVAL                                         # rows of whole chunks
    assert fused(pay=A + 4) == EINVAL and fused(q=A + 8) == EINVAL               # 16-byte alignment
    assert fused(pay=None) == EINVAL
    assert fused(batch=(1 << 32) // (64 * 256)) == EINVAL                         # blocked codes past 2^32
    assert fused(batch=0) == OK


def test_library_has_no_undefined_internal_symbols():
    # every function the library calls is defined in it or in a system/ROCm
    # library: none of its own namespaces may be left undefined
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", LIB], capture_output=True, text=True).stdout
    bad = [l for l in out.splitlines() if "_GLOBAL__N" in l or "_ZN2hq" in l]
    assert not bad, bad
