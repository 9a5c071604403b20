"""ctypes wrapper of the CPU oracle (``hq_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke``
and the CPU-baseline leg of ``bench.py``; never by the product package.
It shares no code with the HIP library.  Arrays are numpy, host memory.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC = os.path.join(HERE, "hq_oracle.c")

CFLAGS = ["-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-msse2",
          "-mfpmath=sse", "-fPIC", "-shared", "-Wall"]

LATTICES = {"Z": 1, "A2": 2, "D4": 4, "E8": 8}
DIMS = {1: 1, 2: 2, 4: 4, 8: 8}
F32, BF16 = 0, 1
OK, EINVAL, ENOSPC, ENONFINITE, ECORRUPT = 0, -1, -3, -4, -5
CHUNK_TILES = 64


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C99, no contraction, no fast-math)."""
    stale = not os.path.exists(LIB_PATH) or any(
        os.path.getmtime(f) > os.path.getmtime(LIB_PATH) for f in (SRC, os.path.join(HERE, "hq_oracle.h")))
    if force or stale:
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Params(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_uint32), ("tile", ctypes.c_uint32),
                ("rows", ctypes.c_uint64), ("cols", ctypes.c_uint64),
                ("lattice", ctypes.c_uint32), ("dither", ctypes.c_uint32),
                ("c", ctypes.c_float), ("pad_", ctypes.c_uint32),
                ("seed", ctypes.c_uint64), ("tile_base", ctypes.c_uint64)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp = ctypes.c_void_p
        L.hqo_pcg_hash.argtypes = [ctypes.c_uint32]; L.hqo_pcg_hash.restype = ctypes.c_uint32
        L.hqo_key.argtypes = [ctypes.c_uint64, ctypes.c_uint32]; L.hqo_key.restype = ctypes.c_uint32
        L.hqo_sign_bit.argtypes = [ctypes.c_uint64, ctypes.c_uint32]; L.hqo_sign_bit.restype = ctypes.c_uint32
        L.hqo_dither_bits.argtypes = [ctypes.c_uint64, ctypes.c_uint32]; L.hqo_dither_bits.restype = ctypes.c_uint32
        L.hqo_rht_forward.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint64, vp]; L.hqo_rht_forward.restype = None
        L.hqo_rht_inverse.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint64, vp]; L.hqo_rht_inverse.restype = None
        L.hqo_tile_step.argtypes = [vp, ctypes.c_uint32, ctypes.c_float, P(ctypes.c_int)]
        L.hqo_tile_step.restype = ctypes.c_float
        L.hqo_nearest.argtypes = [ctypes.c_uint32, vp, vp, vp]; L.hqo_nearest.restype = None
        L.hqo_nearest_batch.argtypes = [ctypes.c_uint32, vp, ctypes.c_uint64, vp, vp]
        L.hqo_nearest_batch.restype = None
        L.hqo_dither_block.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_uint32, vp]
        L.hqo_dither_block.restype = None
        L.hqo_zigzag.argtypes = [ctypes.c_int32]; L.hqo_zigzag.restype = ctypes.c_uint32
        L.hqo_unzigzag.argtypes = [ctypes.c_uint32]; L.hqo_unzigzag.restype = ctypes.c_int32
        L.hqo_rice_k.argtypes = [vp, ctypes.c_uint32]; L.hqo_rice_k.restype = ctypes.c_uint32
        L.hqo_rice_cost.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint32]; L.hqo_rice_cost.restype = ctypes.c_uint64
        L.hqo_tile_bound_bits.argtypes = [P(_Params)]; L.hqo_tile_bound_bits.restype = ctypes.c_uint32
        L.hqo_payload_cap_words.argtypes = [P(_Params)]; L.hqo_payload_cap_words.restype = ctypes.c_uint64
        L.hqo_encode.argtypes = [vp, P(_Params), vp, vp, vp, vp, ctypes.c_uint64]
        L.hqo_encode.restype = ctypes.c_int
        L.hqo_decode.argtypes = [vp, vp, vp, vp, ctypes.c_uint64, P(_Params), vp]
        L.hqo_decode.restype = ctypes.c_int
        L.hqo_encode_tiles.argtypes = [vp, P(_Params), ctypes.c_uint64, ctypes.c_uint64, vp, vp, vp,
                                       ctypes.c_uint64]
        L.hqo_encode_tiles.restype = ctypes.c_int
        L.hqo_decode_tiles.argtypes = [vp, vp, vp, ctypes.c_uint64, P(_Params), ctypes.c_uint64, ctypes.c_uint64, vp]
        L.hqo_decode_tiles.restype = ctypes.c_int
        L.hqo_rotate.argtypes = [vp, ctypes.c_uint32, ctypes.c_uint32, vp, ctypes.c_uint32, ctypes.c_uint64, vp,
                                 ctypes.c_uint32]
        L.hqo_rotate.restype = None
        L.hqo_decode_codes.argtypes = [vp, vp, vp, vp, ctypes.c_uint64, P(_Params), vp, P(ctypes.c_uint32)]
        L.hqo_decode_codes.restype = ctypes.c_int
        L.hqo_act_quant.argtypes = [vp, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64, vp, vp]
        L.hqo_act_quant.restype = None
        L.hqo_codes_matmul.argtypes = [vp, vp, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32, vp, vp,
                                       ctypes.c_uint64, vp]
        L.hqo_codes_matmul.restype = None
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def params(rows, cols, tile, lattice, c, seed, dtype=BF16, dither=0, tile_base=0) -> _Params:
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    return _Params(dtype=dtype, tile=tile, rows=rows, cols=cols, lattice=lat,
                   dither=int(dither), c=float(np.float32(c)), pad_=0, seed=seed, tile_base=tile_base)


@dataclass
class Encoded:
    step: np.ndarray       # uint16 [T] (bf16 bits)
    meta: np.ndarray       # uint16 [T] (len << 3 | k)
    chunk_off: np.ndarray  # uint32 [C+1] (word offsets)
    payload: np.ndarray    # uint32 [chunk_off[-1]]
    status: int


# ---------------------------------------------------------------- steps
def pcg_hash(v: int) -> int:
    return lib().hqo_pcg_hash(v & 0xFFFFFFFF)


def sign_bits(seed: int, n: int) -> np.ndarray:
    return np.array([lib().hqo_sign_bit(seed, i) for i in range(n)], dtype=np.uint32)


def dither_bits(seed: int, g: int) -> int:
    return lib().hqo_dither_bits(seed, g)


def rht_forward(x: np.ndarray, seed: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty_like(x)
    lib().hqo_rht_forward(_ptr(x), x.size, seed, _ptr(y))
    return y


def rht_inverse(y: np.ndarray, seed: int) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    x = np.empty_like(y)
    lib().hqo_rht_inverse(_ptr(y), y.size, seed, _ptr(x))
    return x


def tile_step(y: np.ndarray, c: float):
    y = np.ascontiguousarray(y, dtype=np.float32)
    nf = ctypes.c_int(0)
    s = lib().hqo_tile_step(_ptr(y), y.size, float(np.float32(c)), ctypes.byref(nf))
    return np.float32(s), bool(nf.value)


def nearest(lattice, t: np.ndarray):
    """Nearest lattice point of one block; returns (code[0]=coset bit, ints, point)."""
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    t = np.ascontiguousarray(t, dtype=np.float32)
    code = np.zeros(9, dtype=np.int32)
    pt = np.zeros(8, dtype=np.float32)
    lib().hqo_nearest(lat, _ptr(t), _ptr(code), _ptr(pt))
    d = DIMS[lat]
    return int(code[0]), code[1:1 + d].copy(), pt[:d].copy()


def nearest_batch(lattice, t: np.ndarray):
    """t: [nblocks, d] float32 -> (coset bits [nblocks], ints [nblocks, d], points [nblocks, d])."""
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    d = DIMS[lat]
    t = np.ascontiguousarray(t, dtype=np.float32).reshape(-1, d)
    nb = t.shape[0]
    codes = np.zeros((nb, d + 1), np.int32)
    pts = np.zeros((nb, d), np.float32)
    lib().hqo_nearest_batch(lat, _ptr(t), nb, _ptr(codes), _ptr(pts))
    return codes[:, 0].copy(), codes[:, 1:].copy(), pts


def dither_block(lattice, seed: int, g0: int) -> np.ndarray:
    lat = LATTICES[lattice] if isinstance(lattice, str) else int(lattice)
    u = np.zeros(8, dtype=np.float32)
    lib().hqo_dither_block(lat, seed, g0, _ptr(u))
    return u[:DIMS[lat]].copy()


def rice_k(u: np.ndarray) -> int:
    u = np.ascontiguousarray(u, dtype=np.uint32)
    return lib().hqo_rice_k(_ptr(u), u.size)


def rice_cost(u: np.ndarray, k: int) -> int:
    u = np.ascontiguousarray(u, dtype=np.uint32)
    return lib().hqo_rice_cost(_ptr(u), u.size, k)


def zigzag(v: int) -> int:
    return lib().hqo_zigzag(v)


def unzigzag(u: int) -> int:
    return lib().hqo_unzigzag(u)


def tile_bound_bits(p: _Params) -> int:
    return lib().hqo_tile_bound_bits(ctypes.byref(p))


# ---------------------------------------------------------------- path
def _as_input(x: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        assert x.dtype == np.float32
    else:
        assert x.dtype == np.uint16, "bf16 input is passed as uint16 bit patterns"
    return np.ascontiguousarray(x)


def encode(x: np.ndarray, tile: int, lattice, c: float, seed: int, dither: int = 0, tile_base: int = 0) -> Encoded:
    """x: 2-D float32 array, or uint16 array holding bf16 bit patterns.  With
    tile_base, x is the slice of tiles [tile_base, ...) of a larger tensor
    (the dither is indexed by the global coordinate)."""
    dtype = F32 if x.dtype == np.float32 else BF16
    x = _as_input(x, dtype)
    rows, cols = x.shape
    p = params(rows, cols, tile, lattice, c, seed, dtype, dither, tile_base)
    cap = lib().hqo_payload_cap_words(ctypes.byref(p))
    if cap == 0:
        raise ValueError("configuration rejected by the oracle")
    T = rows * cols // tile
    C = (T + CHUNK_TILES - 1) // CHUNK_TILES
    step = np.zeros(T, np.uint16)
    meta = np.zeros(T, np.uint16)
    off = np.zeros(C + 1, np.uint32)
    pay = np.zeros(cap, np.uint32)
    st = lib().hqo_encode(_ptr(x), ctypes.byref(p), _ptr(step), _ptr(meta), _ptr(off), _ptr(pay), cap)
    if st not in (OK, ENONFINITE):
        raise RuntimeError(f"oracle encode failed: {st}")
    return Encoded(step, meta, off, pay[: off[-1]].copy(), st)


def decode(e: Encoded, rows: int, cols: int, tile: int, lattice, c: float, seed: int,
           dtype: int = F32, dither: int = 0, tile_base: int = 0):
    """Returns (x_hat, status); x_hat float32, or uint16 bf16 bits if dtype == BF16."""
    p = params(rows, cols, tile, lattice, c, seed, dtype, dither, tile_base)
    out = np.zeros((rows, cols), np.float32 if dtype == F32 else np.uint16)
    pay = np.ascontiguousarray(e.payload, dtype=np.uint32)
    if pay.size == 0:
        pay = np.zeros(1, np.uint32)
    st = lib().hqo_decode(_ptr(np.ascontiguousarray(e.step)), _ptr(np.ascontiguousarray(e.meta)),
                          _ptr(np.ascontiguousarray(e.chunk_off)), _ptr(pay), e.payload.size,
                          ctypes.byref(p), _ptr(out))
    return out, st


def encode_tiles(x: np.ndarray, tile: int, lattice, c: float, seed: int, t0: int, t1: int,
                 dither: int = 0):
    """Tile range [t0, t1) of a full encode: (step, meta, bits) with the tiles'
    bitstreams concatenated from bit 0."""
    dtype = F32 if x.dtype == np.float32 else BF16
    x = _as_input(x, dtype)
    rows, cols = x.shape
    p = params(rows, cols, tile, lattice, c, seed, dtype, dither)
    bound = lib().hqo_tile_bound_bits(ctypes.byref(p))
    cap = ((t1 - t0) * bound + 31) // 32 + 1
    step = np.zeros(t1 - t0, np.uint16)
    meta = np.zeros(t1 - t0, np.uint16)
    bits = np.zeros(cap, np.uint32)
    st = lib().hqo_encode_tiles(_ptr(x), ctypes.byref(p), t0, t1, _ptr(step), _ptr(meta), _ptr(bits), cap)
    if st not in (OK, ENONFINITE):
        raise RuntimeError(f"oracle encode_tiles failed: {st}")
    return step, meta, bits


def decode_tiles(step, meta, bits, rows, cols, tile, lattice, c, seed, t0, t1, dtype=F32, dither=0):
    """Decode tiles [t0, t1) of a tensor of shape (rows, cols) from their
    concatenated bitstreams; returns ([(t1 - t0) * tile] array, status)."""
    p = params(rows, cols, tile, lattice, c, seed, dtype, dither)
    out = np.zeros((t1 - t0) * tile, np.float32 if dtype == F32 else np.uint16)
    bits = np.ascontiguousarray(bits, np.uint32)
    st = lib().hqo_decode_tiles(_ptr(np.ascontiguousarray(step, np.uint16)),
                                _ptr(np.ascontiguousarray(meta, np.uint16)), _ptr(bits), bits.size,
                                ctypes.byref(p), t0, t1, _ptr(out))
    return out, st


# ---------------------------------------------------------------- closed-loop rate
# The pages claim the realized rate lands within about 0.01 bps of any target
# (gist.science explainer of HyperQuant, Methodology section 3, "Bit-Stripping
# and Rice Coding").  The frozen table reaches that on Gaussian data; on a
# given tensor the constant c is found by bisection instead, each step one
# full encode at a trial c.  The rate is that of the stored stream,
# 32 * payload words / scalars (coset and Rice bits plus the word alignment
# of each 64-tile chunk).
#
# The bracket around the high-rate step constant of an entropy-coded lattice
# quantiser, c = sqrt(2 pi e) 2^-R V^(-1/d) (V the covolume: Z 1, A2 sqrt3/2,
# D4 2, E8 1), is K_lattice 2^-floor(R) scaled by 2^-3 and 2^2 (exact fp32
# products), with K = fl32(sqrt(2 pi e) V^(-1/d)) stored as its bits.
RATE_K_BITS = {"Z": 0x40843F56, "A2": 0x408E1BED, "D4": 0x405E69A9, "E8": 0x40843F56}
RATE_TOL = 0.01
RATE_ITERS = 30


def rate_bracket(lattice: str, target: float) -> tuple:
    k = float(np.array([RATE_K_BITS[lattice]], np.uint32).view(np.float32)[0])
    e = math.floor(float(np.float32(target)))
    return float(np.float32(k * 2.0 ** (-e - 3))), float(np.float32(k * 2.0 ** (-e + 2)))


def stream_bps(e: Encoded, numel: int) -> float:
    return 32.0 * int(e.chunk_off[-1]) / numel


def rate_search(x: np.ndarray, tile: int, lattice: str, target: float, seed: int, dither: int = 0):
    """Bisection on c over the bracket, at the geometric midpoint
    fl32(sqrt(lo * hi)) (the product is exact in fp64): more bits than the
    target moves lo up, fewer moves hi down.  Stops when the stream rate is
    within RATE_TOL of the target, when the midpoint equals an end (fp32
    resolution), or after RATE_ITERS encodes.  Returns (c, rate, encodes,
    Encoded of the last trial)."""
    target = float(np.float32(target))
    lo, hi = rate_bracket(lattice, target)
    numel = x.size
    for it in range(1, RATE_ITERS + 1):
        c = float(np.float32(math.sqrt(lo * hi)))
        e = encode(x, tile, lattice, c, seed, dither)
        r = stream_bps(e, numel)
        if abs(r - target) <= RATE_TOL or c == lo or c == hi:
            break
        if r > target:
            lo = c
        else:
            hi = c
    return c, r, it, e


# ---------------------------------------------------------------- KV rotation
def rotate(Q: np.ndarray, x: np.ndarray, transpose: bool = False, out_dtype: int = F32) -> np.ndarray:
    """y = Q x (or Q^T x) for every d-vector row of x (float32, or uint16 bf16
    bits); Q float32 [d][d].  Returns float32, or uint16 bf16 bits."""
    Q = np.ascontiguousarray(Q, np.float32)
    d = Q.shape[0]
    assert Q.shape == (d, d) and x.shape[-1] == d
    xdt = F32 if x.dtype == np.float32 else BF16
    x = _as_input(x.reshape(-1, d), xdt)
    y = np.zeros(x.shape, np.float32 if out_dtype == F32 else np.uint16)
    lib().hqo_rotate(_ptr(Q), d, int(transpose), _ptr(x), xdt, x.shape[0], _ptr(y), out_dtype)
    return y


# ---------------------------------------------------------------- int8 product path
def decode_codes(e: Encoded, rows: int, cols: int, tile: int, lattice, c: float, seed: int):
    """A stream's integer codes 2P as int8 [rows][cols]: (codes, status, range_flag)."""
    p = params(rows, cols, tile, lattice, c, seed, F32, 0)
    codes = np.zeros((rows, cols), np.int8)
    pay = np.ascontiguousarray(e.payload, dtype=np.uint32)
    if pay.size == 0:
        pay = np.zeros(1, np.uint32)
    flag = ctypes.c_uint32(0)
    st = lib().hqo_decode_codes(_ptr(np.ascontiguousarray(e.step)), _ptr(np.ascontiguousarray(e.meta)),
                                _ptr(np.ascontiguousarray(e.chunk_off)), _ptr(pay), e.payload.size,
                                ctypes.byref(p), _ptr(codes), ctypes.byref(flag))
    return codes, st, flag.value


def act_quant(x: np.ndarray, tile: int, seed: int):
    """Per-tile RHT of activations x [batch][cols] (fp32) in int8 with fp32 scales."""
    x = np.ascontiguousarray(x, np.float32)
    B, cols = x.shape
    q = np.zeros((B, cols), np.int8)
    sc = np.zeros((B, cols // tile), np.float32)
    lib().hqo_act_quant(_ptr(x), B, cols, tile, seed, _ptr(q), _ptr(sc))
    return q, sc


def codes_matmul(codes: np.ndarray, step: np.ndarray, tile: int, q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """y [batch][rows] from the weight codes [rows][cols], tile steps and int8 activations."""
    rows, cols = codes.shape
    B = q.shape[0]
    y = np.zeros((B, rows), np.float32)
    lib().hqo_codes_matmul(_ptr(np.ascontiguousarray(codes)), _ptr(np.ascontiguousarray(step, np.uint16)), rows,
                           cols, tile, _ptr(np.ascontiguousarray(q)), _ptr(np.ascontiguousarray(scale, np.float32)),
                           B, _ptr(y))
    return y
