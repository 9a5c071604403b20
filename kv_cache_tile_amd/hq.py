"""Thin Python binding of libhq.so (argument marshalling only).

Every step of the codec runs in the library's HIP kernels; torch provides the
device memory and the stream.  Function names follow the C ABI (include/hq.h):
``encode`` / ``decode`` (weights) and ``kv_encode`` / ``kv_decode`` (KV cache).
Importing this module on a machine without the built library or without a GPU
raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhq.so")

LATTICES = {"Z": 1, "A2": 2, "D4": 4, "E8": 8}
F32, BF16 = 0, 1
FLAG_NONFINITE, FLAG_CORRUPT, FLAG_NOSPACE, FLAG_RANGE, FLAG_STALL = 1, 2, 4, 8, 16
CHUNK_TILES = 64

EXPORTS = ("hq_plan", "hq_encode", "hq_decode", "hq_kv_encode", "hq_kv_decode", "hq_strerror",
           "hq_version", "hq_plan_c", "hq_encode_c", "hq_decode_c", "hq_rate_bracket", "hq_encode_rate",
           "hq_encode_length_c", "hq_rotate", "hq_decode_codes", "hq_act_quant",
           "hq_act_quant_blocked", "hq_codes_matmul", "hq_nearest", "hq_encode_c_noalloc", "hq_codes_matmul_fused")


class HQError(RuntimeError):
    pass


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise HQError(f"{LIB_PATH} is missing: run `python -m kv_cache_tile_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        u32, u64, vp, f32 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_float
        P = ctypes.POINTER
        L.hq_plan.argtypes = [u32, u64, u64, u32, u32, f32, u32, P(u64), P(u64), P(u64), P(u64), P(u32), P(f32)]
        L.hq_plan.restype = ctypes.c_int
        enc = [vp, u32, u64, u64, u32, u32, f32, u64, vp, u64, vp, vp, vp, vp, vp, u64, vp]
        L.hq_encode.argtypes = enc
        L.hq_encode.restype = ctypes.c_int
        L.hq_kv_encode.argtypes = [vp, u32, u64, u32, u32, f32, u64, vp, u64, vp, vp, vp, vp, vp, u64, vp]
        L.hq_kv_encode.restype = ctypes.c_int
        L.hq_decode.argtypes = [vp, u64, vp, vp, vp, u32, u64, u64, u32, u32, f32, u64, vp, vp, vp]
        L.hq_decode.restype = ctypes.c_int
        L.hq_kv_decode.argtypes = [vp, u64, vp, vp, vp, u32, u64, u32, u32, f32, u64, vp, vp, vp]
        L.hq_kv_decode.restype = ctypes.c_int
        L.hq_plan_c.argtypes = [u32, u64, u64, u32, u32, f32, u32, P(u64), P(u64), P(u64), P(u64), P(u32)]
        L.hq_plan_c.restype = ctypes.c_int
        L.hq_encode_c.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, u64, vp, vp, vp, vp, vp, u64, vp]
        L.hq_encode_c.restype = ctypes.c_int
        L.hq_encode_c_noalloc.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, u64, vp, vp, vp, vp, vp]
        L.hq_encode_c_noalloc.restype = ctypes.c_int
        L.hq_decode_c.argtypes = [vp, u64, vp, vp, vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, vp, vp]
        L.hq_decode_c.restype = ctypes.c_int
        L.hq_rate_bracket.argtypes = [u32, f32, P(f32), P(f32)]
        L.hq_rate_bracket.restype = ctypes.c_int
        L.hq_encode_rate.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, u64, vp, vp, vp, vp, vp, u64,
                                     P(f32), P(ctypes.c_double), P(u32), vp]
        L.hq_encode_rate.restype = ctypes.c_int
        L.hq_encode_length_c.argtypes = [vp, u32, u64, u64, u32, u32, f32, u64, u32, vp, vp]
        L.hq_encode_length_c.restype = ctypes.c_int
        L.hq_rotate.argtypes = [vp, u32, u32, vp, u32, u64, vp, u32, vp]
        L.hq_rotate.restype = ctypes.c_int
        L.hq_decode_codes.argtypes = [vp, u64, vp, vp, vp, u64, u64, u32, u32, f32, u64, vp, vp, vp]
        L.hq_decode_codes.restype = ctypes.c_int
        L.hq_act_quant.argtypes = [vp, u32, u64, u64, u32, u64, vp, vp, vp]
        L.hq_act_quant.restype = ctypes.c_int
        L.hq_act_quant_blocked.argtypes = [vp, u32, u64, u64, u32, u64, vp, vp, vp]
        L.hq_act_quant_blocked.restype = ctypes.c_int
        L.hq_codes_matmul.argtypes = [vp, vp, u64, u64, u32, vp, vp, u64, vp, vp, u64, vp]
        L.hq_codes_matmul.restype = ctypes.c_int
        L.hq_codes_matmul_fused.argtypes = [vp, u64, vp, vp, vp, u64, u64, u32, u32, f32, vp, vp, u64, vp, vp, vp]
        L.hq_codes_matmul_fused.restype = ctypes.c_int
        L.hq_nearest.argtypes = [u32, vp, u64, vp, vp]
        L.hq_nearest.restype = ctypes.c_int
        L.hq_strerror.argtypes = [ctypes.c_int]
        L.hq_strerror.restype = ctypes.c_char_p
        L.hq_version.argtypes = []
        L.hq_version.restype = u32
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise HQError(f"hq error {rc}: {lib().hq_strerror(rc).decode()}")


@dataclass
class Plan:
    tiles: int
    chunks: int
    payload_cap_words: int
    workspace_bytes: int
    tile_bound_bits: int
    rate_constant: float


def plan(dtype: int, rows: int, cols: int, tile: int, lattice: str, bps: float, kv: bool = False) -> Plan:
    vals = [ctypes.c_uint64() for _ in range(4)]
    tb = ctypes.c_uint32()
    rc_ = ctypes.c_float()
    _check(lib().hq_plan(dtype, rows, cols, tile, LATTICES[lattice], float(bps), int(kv),
                         *[ctypes.byref(v) for v in vals], ctypes.byref(tb), ctypes.byref(rc_)))
    return Plan(vals[0].value, vals[1].value, vals[2].value, vals[3].value, tb.value, rc_.value)


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise HQError(f"unsupported dtype {t}")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_workspaces: dict = {}


def workspace(device, nbytes: int) -> torch.Tensor:
    """A zero-initialised encode workspace, reused across the calls made on
    one stream of a device (calls on different streams may overlap in time,
    so each stream has its own)."""
    device = torch.device(device)
    key = (device.index if device.index is not None else torch.cuda.current_device(), _stream(device))
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 16), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


@dataclass
class HQTensor:
    """Compressed tensor: device buffers plus the parameters needed to decode."""
    payload: torch.Tensor     # int32 words (capacity; valid prefix = chunk_off[-1])
    step: torch.Tensor        # int16 bf16 step bits per tile
    meta: torch.Tensor        # int16 (len << 3 | k) per tile
    chunk_off: torch.Tensor   # int32 [chunks + 1]
    status: torch.Tensor      # int32 [1] flags
    shape: tuple
    dtype: torch.dtype
    tile: int
    lattice: str
    bps: float
    seed: int
    kv: bool = False
    extra: dict = field(default_factory=dict)
    c: float | None = None    # explicit rate constant (closed-loop or hq_encode_c streams)

    def payload_words(self) -> int:
        return int(self.chunk_off[-1].item())

    def flags(self) -> int:
        return int(self.status.item())

    def bits_payload(self) -> int:
        """coset + Rice bits (sum of the tile lengths)."""
        return int((self.meta.to(torch.int32) & 0xFFFF).__rshift__(3).sum().item())

    def bits_total(self) -> int:
        """everything stored: payload words, step and meta per tile, chunk offsets."""
        return 32 * self.payload_words() + 32 * self.step.numel() + 32 * self.chunk_off.numel()


def _alloc(p: Plan, device) -> tuple:
    payload = torch.empty(p.payload_cap_words, dtype=torch.int32, device=device)
    step = torch.empty(p.tiles, dtype=torch.int16, device=device)
    meta = torch.empty(p.tiles, dtype=torch.int16, device=device)
    off = torch.empty(p.chunks + 1, dtype=torch.int32, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    return payload, step, meta, off, status


def encode(x: torch.Tensor, tile: int = 128, lattice: str = "E8", bps: float = 4.0, seed: int = 0,
           out: HQTensor | None = None, zero_status: bool = True) -> HQTensor:
    """Encode a 2-D (or any, viewed as [-1, last]) weight tensor on its GPU.
    With `out`, its buffers are reused (and its status word is cleared first
    unless zero_status is False, in which case flags accumulate)."""
    if not x.is_cuda:
        raise HQError("encode needs a GPU tensor")
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    dt = _dtype_code(x2.dtype)
    rows, cols = x2.shape
    p = plan(dt, rows, cols, tile, lattice, bps, kv=False)
    bufs = (out.payload, out.step, out.meta, out.chunk_off, out.status) if out is not None else _alloc(p, x.device)
    payload, step, meta, off, status = bufs
    if out is not None and zero_status:
        status.zero_()
    ws = workspace(x.device, p.workspace_bytes)
    _check(lib().hq_encode(x2.data_ptr(), dt, rows, cols, tile, LATTICES[lattice], float(bps), seed,
                           payload.data_ptr(), payload.numel(), step.data_ptr(), meta.data_ptr(),
                           off.data_ptr(), status.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)))
    if out is not None:
        return out
    return HQTensor(payload, step, meta, off, status, tuple(x.shape), x.dtype, tile, lattice, float(bps),
                    seed, False)


def decode(h: HQTensor, out: torch.Tensor | None = None) -> torch.Tensor:
    rows = 1
    for s in h.shape[:-1]:
        rows *= s
    cols = h.shape[-1]
    if out is None:
        out = torch.empty(h.shape, dtype=h.dtype, device=h.payload.device)
    dt = _dtype_code(h.dtype)
    if h.c is not None:
        _check(lib().hq_decode_c(h.payload.data_ptr(), h.payload.numel(), h.step.data_ptr(), h.meta.data_ptr(),
                                 h.chunk_off.data_ptr(), dt, rows, cols, h.tile, LATTICES[h.lattice], h.c, h.seed,
                                 int(h.kv), out.data_ptr(), h.status.data_ptr(), _stream(out.device)))
        return out
    fn = lib().hq_kv_decode if h.kv else lib().hq_decode
    if h.kv:
        rc = fn(h.payload.data_ptr(), h.payload.numel(), h.step.data_ptr(), h.meta.data_ptr(),
                h.chunk_off.data_ptr(), dt, rows, cols, LATTICES[h.lattice], h.bps, h.seed, out.data_ptr(),
                h.status.data_ptr(), _stream(out.device))
    else:
        rc = fn(h.payload.data_ptr(), h.payload.numel(), h.step.data_ptr(), h.meta.data_ptr(),
                h.chunk_off.data_ptr(), dt, rows, cols, h.tile, LATTICES[h.lattice], h.bps, h.seed,
                out.data_ptr(), h.status.data_ptr(), _stream(out.device))
    _check(rc)
    return out


def kv_encode(x: torch.Tensor, lattice: str = "E8", bps: float = 2.0, seed: int = 0,
              out: HQTensor | None = None) -> HQTensor:
    """Encode KV vectors: x[..., head_dim], one tile per (token, head) vector, dithered."""
    if not x.is_cuda:
        raise HQError("kv_encode needs a GPU tensor")
    hd = x.shape[-1]
    x2 = x.reshape(-1, hd).contiguous()
    dt = _dtype_code(x2.dtype)
    tokens = x2.shape[0]
    p = plan(dt, tokens, hd, hd, lattice, bps, kv=True)
    bufs = (out.payload, out.step, out.meta, out.chunk_off, out.status) if out is not None else _alloc(p, x.device)
    payload, step, meta, off, status = bufs
    if out is not None:
        status.zero_()
    ws = workspace(x.device, p.workspace_bytes)
    _check(lib().hq_kv_encode(x2.data_ptr(), dt, tokens, hd, LATTICES[lattice], float(bps), seed,
                              payload.data_ptr(), payload.numel(), step.data_ptr(), meta.data_ptr(),
                              off.data_ptr(), status.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)))
    if out is not None:
        return out
    return HQTensor(payload, step, meta, off, status, tuple(x.shape), x.dtype, hd, lattice, float(bps), seed,
                    True)


def kv_decode(h: HQTensor, out: torch.Tensor | None = None) -> torch.Tensor:
    if not h.kv:
        raise HQError("not a KV tensor")
    return decode(h, out)


# ---------------------------------------------------------------- explicit constant, closed-loop rate
def plan_c(dtype: int, rows: int, cols: int, tile: int, lattice: str, c: float, kv: bool = False) -> Plan:
    vals = [ctypes.c_uint64() for _ in range(4)]
    tb = ctypes.c_uint32()
    _check(lib().hq_plan_c(dtype, rows, cols, tile, LATTICES[lattice], float(c), int(kv),
                           *[ctypes.byref(v) for v in vals], ctypes.byref(tb)))
    return Plan(vals[0].value, vals[1].value, vals[2].value, vals[3].value, tb.value, float(c))


def rate_bracket(lattice: str, target_bps: float) -> tuple:
    lo, hi = ctypes.c_float(), ctypes.c_float()
    _check(lib().hq_rate_bracket(LATTICES[lattice], float(target_bps), ctypes.byref(lo), ctypes.byref(hi)))
    return lo.value, hi.value


def _rows_cols(x: torch.Tensor, tile: int, kv: bool):
    if not x.is_cuda:
        raise HQError("needs a GPU tensor")
    x2 = x.reshape(-1, tile if kv else x.shape[-1]).contiguous()
    return x2, x2.shape[0], x2.shape[1]


def encode_c(x: torch.Tensor, tile: int, lattice: str, c: float, seed: int = 0, kv: bool = False,
             out: HQTensor | None = None, zero_status: bool = True) -> HQTensor:
    """Encode with an explicit rate constant c (step = bf16(rms * c)); KV: tile = head_dim.
    With `out` (for instance the result of encode_rate on this tensor), its
    buffers are reused and it is returned with its constant set to c."""
    x2, rows, cols = _rows_cols(x, tile, kv)
    dt = _dtype_code(x2.dtype)
    p = plan_c(dt, rows, cols, tile, lattice, c, kv)
    if out is not None:
        payload, step, meta, off, status = out.payload, out.step, out.meta, out.chunk_off, out.status
        if zero_status:
            status.zero_()
    else:
        payload, step, meta, off, status = _alloc(p, x.device)
    ws = workspace(x.device, p.workspace_bytes)
    _check(lib().hq_encode_c(x2.data_ptr(), dt, rows, cols, tile, LATTICES[lattice], float(c), seed, int(kv),
                             payload.data_ptr(), payload.numel(), step.data_ptr(), meta.data_ptr(), off.data_ptr(),
                             status.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)))
    if out is not None:
        out.c = float(c)
        return out
    return HQTensor(payload, step, meta, off, status, tuple(x.shape), x.dtype, tile, lattice, float("nan"), seed,
                    kv, c=float(c))


def encode_c_noalloc(x: torch.Tensor, tile: int, lattice: str, c: float, seed: int, out: HQTensor,
                     kv: bool = False) -> HQTensor:
    """encode_c into the buffers of `out` (sized for this tensor and c), with
    the library's static workspace: no device allocation anywhere in the call."""
    x2, rows, cols = _rows_cols(x, tile, kv)
    _check(lib().hq_encode_c_noalloc(x2.data_ptr(), _dtype_code(x2.dtype), rows, cols, tile, LATTICES[lattice],
                                     float(c), seed, int(kv), out.payload.data_ptr(), out.payload.numel(),
                                     out.step.data_ptr(), out.meta.data_ptr(), out.chunk_off.data_ptr(),
                                     out.status.data_ptr(), _stream(x.device)))
    out.c = float(c)
    return out


def encode_length_c(x: torch.Tensor, tile: int, lattice: str, c: float, seed: int = 0, kv: bool = False,
                    out: torch.Tensor | None = None) -> torch.Tensor:
    """The length pass: the payload word count (chunk_off[C]) that encode_c
    with these arguments would produce, as a device int64 tensor of one
    element, without writing a stream.  With `out` (a zeroed device int64
    scalar), the count is added to it."""
    x2, rows, cols = _rows_cols(x, tile, kv)
    words = torch.zeros((), dtype=torch.int64, device=x.device) if out is None else out
    _check(lib().hq_encode_length_c(x2.data_ptr(), _dtype_code(x2.dtype), rows, cols, tile, LATTICES[lattice],
                                    float(c), seed, int(kv), words.data_ptr(), _stream(x.device)))
    return words


def encode_rate(x: torch.Tensor, tile: int, lattice: str, target_bps: float, seed: int = 0,
                kv: bool = False) -> HQTensor:
    """Closed-loop rate: the library bisects on c, each trial a length pass,
    until the stream would be within 0.01 bits per scalar of target_bps, and
    then encodes it once (synchronous).  The result records c, the rate
    reached and the number of trials (`encodes`) in `extra`."""
    x2, rows, cols = _rows_cols(x, tile, kv)
    dt = _dtype_code(x2.dtype)
    lo, _ = rate_bracket(lattice, target_bps)
    p = plan_c(dt, rows, cols, tile, lattice, lo, kv)
    payload, step, meta, off, status = _alloc(p, x.device)
    ws = workspace(x.device, p.workspace_bytes)
    c, r, n = ctypes.c_float(), ctypes.c_double(), ctypes.c_uint32()
    _check(lib().hq_encode_rate(x2.data_ptr(), dt, rows, cols, tile, LATTICES[lattice], float(target_bps), seed,
                                int(kv), payload.data_ptr(), payload.numel(), step.data_ptr(), meta.data_ptr(),
                                off.data_ptr(), status.data_ptr(), ws.data_ptr(), ws.numel(), ctypes.byref(c),
                                ctypes.byref(r), ctypes.byref(n), _stream(x.device)))
    return HQTensor(payload, step, meta, off, status, tuple(x.shape), x.dtype, tile, lattice, float(target_bps),
                    seed, kv, extra=dict(rate=r.value, encodes=n.value), c=c.value)


# ---------------------------------------------------------------- KV Haar rotation
def rotate(Q: torch.Tensor, x: torch.Tensor, transpose: bool = False, out_dtype: torch.dtype | None = None,
           out: torch.Tensor | None = None) -> torch.Tensor:
    """y = Q x (or Q^T x) for every d-vector (last dim) of x; Q fp32 [d][d] on
    the same GPU, d = 64 or 128."""
    if not x.is_cuda or not Q.is_cuda or Q.dtype != torch.float32:
        raise HQError("rotate needs GPU tensors and an fp32 Q")
    d = Q.shape[0]
    x2 = x.reshape(-1, d).contiguous()
    Qc = Q.contiguous()
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype or x.dtype, device=x.device)
    _check(lib().hq_rotate(Qc.data_ptr(), d, int(transpose), x2.data_ptr(), _dtype_code(x2.dtype), x2.shape[0],
                           out.data_ptr(), _dtype_code(out.dtype), _stream(x.device)))
    return out


def kv_encode_haar(x: torch.Tensor, Q: torch.Tensor, lattice: str = "E8", bps: float = 2.0,
                   seed: int = 0) -> HQTensor:
    """KV vectors rotated by the caller's Haar matrix Q (fp32, rotated values
    kept in fp32), then coded by the dithered KV path; decode with
    kv_decode_haar."""
    y = rotate(Q, x, out_dtype=torch.float32)
    h = kv_encode(y, lattice, bps, seed)
    h.extra["haar_Q"] = Q
    h.extra["haar_out_dtype"] = x.dtype
    return h


def kv_decode_haar(h: HQTensor, out: torch.Tensor | None = None) -> torch.Tensor:
    y = kv_decode(h)
    return rotate(h.extra["haar_Q"], y, transpose=True, out_dtype=h.extra["haar_out_dtype"], out=out)


# ---------------------------------------------------------------- int8 product path
def _rows_cols_c(h: HQTensor) -> tuple:
    if h.kv:
        raise HQError("integer codes: weights only (the KV path is dithered)")
    rows = 1
    for s_ in h.shape[:-1]:
        rows *= s_
    cols = h.shape[-1]
    c = h.c if h.c is not None else plan(_dtype_code(h.dtype), rows, cols, h.tile, h.lattice, h.bps).rate_constant
    return rows, cols, c


def decode_codes(h: HQTensor, out: torch.Tensor | None = None, status: torch.Tensor | None = None) -> torch.Tensor:
    """The weights' integer codes 2P (int8 [rows][cols]) for hq_codes_matmul;
    flags go to `status` (default: the stream's own status word)."""
    rows, cols, c = _rows_cols_c(h)
    if out is None:
        out = torch.empty((rows, cols), dtype=torch.int8, device=h.payload.device)
    st = h.status if status is None else status
    _check(lib().hq_decode_codes(h.payload.data_ptr(), h.payload.numel(), h.step.data_ptr(), h.meta.data_ptr(),
                                 h.chunk_off.data_ptr(), rows, cols, h.tile, LATTICES[h.lattice], c, h.seed,
                                 out.data_ptr(), st.data_ptr(), _stream(out.device)))
    return out


def fused_supported(h: HQTensor) -> bool:
    """Whether codes_matmul_fused takes this stream: Z, D4 or E8 weights whose
    rows are whole 64-tile chunks."""
    return not h.kv and h.lattice != "A2" and h.shape[-1] % (CHUNK_TILES * h.tile) == 0


def codes_matmul_fused(h: HQTensor, q: torch.Tensor, scale: torch.Tensor, status: torch.Tensor,
                       out: torch.Tensor | None = None) -> torch.Tensor:
    """y [batch][rows] = the int8 product straight from the stream (one launch),
    with q, scale = act_quant(x, ..., blocked=True); CORRUPT / RANGE flags go
    to `status`."""
    rows, cols, c = _rows_cols_c(h)
    B = scale.shape[0]
    if q.dim() != 1 or q.numel() != blocked_size(B, cols) or scale.shape != (B, cols // h.tile):
        raise HQError("codes_matmul_fused takes act_quant(x, tile, seed, blocked=True)'s output")
    if out is None:
        out = torch.empty((B, rows), dtype=torch.float32, device=q.device)
    _check(lib().hq_codes_matmul_fused(h.payload.data_ptr(), h.payload.numel(), h.step.data_ptr(),
                                       h.meta.data_ptr(), h.chunk_off.data_ptr(), rows, cols, h.tile,
                                       LATTICES[h.lattice], c, q.data_ptr(), scale.data_ptr(), B, out.data_ptr(),
                                       status.data_ptr(), _stream(q.device)))
    return out


def blocked_size(batch: int, cols: int) -> int:
    """Bytes of act_quant(..., blocked=True)'s codes: batch rounded up to 32, times cols."""
    return (batch + 31) // 32 * 32 * cols


def act_quant(x: torch.Tensor, tile: int, seed: int, out: tuple | None = None, blocked: bool = False) -> tuple:
    """Per-tile RHT of activations x [batch][cols] in int8, with fp32 scales
    (into out = (q, scale) when given).  q is int8 [batch][cols], or with
    blocked=True the flat matrix-core order that codes_matmul_fused reads
    (hq_act_quant_blocked)."""
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    B, cols = x2.shape
    qshape = (blocked_size(B, cols),) if blocked else (B, cols)
    if out is not None:
        q, sc = out
        if q.shape != qshape or q.dtype != torch.int8 or sc.shape != (B, cols // tile) or \
                sc.dtype != torch.float32 or not (q.is_contiguous() and sc.is_contiguous()):
            raise ValueError(f"act_quant: out must be int8 {list(qshape)} and fp32 [batch][cols / tile], contiguous")
    else:
        q = torch.empty(qshape, dtype=torch.int8, device=x.device)
        sc = torch.empty((B, cols // tile), dtype=torch.float32, device=x.device)
    fn = lib().hq_act_quant_blocked if blocked else lib().hq_act_quant
    _check(fn(x2.data_ptr(), _dtype_code(x2.dtype), B, cols, tile, seed, q.data_ptr(), sc.data_ptr(),
              _stream(x.device)))
    return q, sc


def codes_matmul(codes: torch.Tensor, step: torch.Tensor, tile: int, q: torch.Tensor, scale: torch.Tensor,
                 out: torch.Tensor | None = None, work: torch.Tensor | None = None) -> torch.Tensor:
    """y [batch][rows] from int8 weight codes, their tile steps and int8 activations."""
    rows, cols = codes.shape
    B = q.shape[0]
    if out is None:
        out = torch.empty((B, rows), dtype=torch.float32, device=codes.device)
    if work is None:
        work = torch.empty(B * rows * (cols // tile), dtype=torch.int32, device=codes.device)
    _check(lib().hq_codes_matmul(codes.data_ptr(), step.data_ptr(), rows, cols, tile, q.data_ptr(),
                                 scale.data_ptr(), B, out.data_ptr(), work.data_ptr(), 4 * work.numel(),
                                 _stream(codes.device)))
    return out


def matmul_compressed(h: HQTensor, x: torch.Tensor) -> torch.Tensor:
    """x @ W_hat^T for compressed weights h, through the int8 product path
    (fused with the decode where the shape allows).  Synchronises to read its
    own status word, and raises if a tile's codes were saturated (the result
    would not be x W_hat^T) or the stream is corrupt."""
    fused = fused_supported(h)
    q, sc = act_quant(x, h.tile, h.seed, blocked=fused)
    status = torch.zeros(1, dtype=torch.int32, device=q.device)
    if fused:
        y = codes_matmul_fused(h, q, sc, status)
    else:
        y = codes_matmul(decode_codes(h, status=status), h.step, h.tile, q, sc)
    flags = int(status.item())
    if flags & FLAG_RANGE:
        raise HQError("integer codes beyond [-127, 127] were saturated: the product is not x W_hat^T")
    if flags & FLAG_CORRUPT:
        raise HQError("corrupt compressed stream")
    return y


# ---------------------------------------------------------------- the quantiser alone
def nearest(lattice: str, t: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """Nearest lattice points of the d-blocks of t (fp32 [..., d] on a GPU), with
    the encoder's decision and tie rules; returns fp32 points of t's shape."""
    if not t.is_cuda or t.dtype != torch.float32:
        raise HQError("nearest needs an fp32 GPU tensor")
    d = LATTICES[lattice]
    t2 = t.reshape(-1, d).contiguous()
    if out is None:
        out = torch.empty(t.shape, dtype=torch.float32, device=t.device)
    _check(lib().hq_nearest(LATTICES[lattice], t2.data_ptr(), t2.shape[0], out.data_ptr(), _stream(t.device)))
    return out
