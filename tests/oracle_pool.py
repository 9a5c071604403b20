"""The CPU oracle run in parallel host processes, for full-tensor parity.

Test infrastructure only.  Tiles are independent, the sign diagonal depends
only on the seed and the dither on the global coordinate, so a chunk-aligned
slice of tiles [t0, t1) of a tensor is encoded and decoded by the oracle as a
tensor of its own (tile_base = t0): its stream is the whole tensor's stream
between chunk offsets t0/64 and t1/64 (offsets taken relative to the first),
and its reconstruction is the whole one's rows.  Workers are spawned
processes that import numpy and the oracle (never the GPU); a slice's input
is either sent to them or drawn by them from the seeded generators.
"""
from __future__ import annotations

import multiprocessing as mp
import os

import numpy as np

CHUNK = 64


def worker_count() -> int:
    """Host processes for the oracle: the CPUs this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def make_pool(n: int | None = None):
    return mp.get_context("spawn").Pool(n or worker_count())


def _input(spec):
    """The slice's input: ("array", x) as given; ("kv", which, b) batch entry b
    of the KV cache configuration as bf16 bits [H * S, D]; ("dit", layer) a
    layer of the DiT stack as bf16 bits."""
    from kv_cache_tile_amd import workloads
    kind = spec[0]
    if kind == "array":
        return spec[1]
    if kind == "kv":
        c = workloads.CONFIGS[3]
        x = workloads.kv_cache_entry(spec[2], c["heads"], c["seq"], c["head_dim"], key=3, which=spec[1])
        return workloads.bf16_bits(workloads.to_bf16(x.reshape(-1, c["head_dim"])))
    if kind == "dit":
        c = workloads.CONFIGS[4]
        return workloads.bf16_bits(workloads.to_bf16(workloads.dit_layer(c["rows"], c["cols"], key=4, layer=spec[1])))
    raise ValueError(kind)


def draw_input(spec):
    """Only the input of a slice (a worker draws it)."""
    return _input(spec)


def oracle_slice(task):
    """One slice through the oracle: encode, then decode of its own stream.
    task = (spec, tile, lattice, c, seed, dither, tile_base, want_x).  Returns
    the stream, the reconstruction's bits and the two statuses (and the input
    when asked)."""
    spec, tile, lattice, c, seed, dither, tile_base, want_x = task
    import oracle
    x = _input(spec)
    x2 = x.reshape(-1, tile) if dither else x.reshape(-1, x.shape[-1])
    e = oracle.encode(x2, tile, lattice, c, seed, dither, tile_base)
    out_dtype = oracle.F32 if x2.dtype == np.float32 else oracle.BF16
    xh, dst = oracle.decode(e, x2.shape[0], x2.shape[1], tile, lattice, c, seed, out_dtype, dither, tile_base)
    bits = xh.view(np.uint32) if xh.dtype == np.float32 else xh.view(np.uint16)
    r = dict(step=e.step, meta=e.meta, off=e.chunk_off, payload=e.payload, out=bits.reshape(-1),
             status=e.status, dstatus=dst)
    if want_x:
        r["x"] = x
    return r


def chunk_slices(T: int, parts: int):
    """[t0, t1) tile ranges on chunk boundaries, about `parts` of them."""
    C = (T + CHUNK - 1) // CHUNK
    per = max(1, (C + parts - 1) // parts)
    return [(CHUNK * c0, min(T, CHUNK * (c0 + per))) for c0 in range(0, C, per)]


def compare_slice(gpu: dict, t0: int, t1: int, tile: int, ora: dict, ok_status: int, label: str):
    """The GPU's full-tensor arrays (step, meta, off, payload, out as host
    numpy) against the oracle's stream of tiles [t0, t1), element by element."""
    c0, c1 = t0 // CHUNK, (t1 + CHUNK - 1) // CHUNK
    np.testing.assert_array_equal(gpu["step"][t0:t1], ora["step"], err_msg=f"{label}: step")
    np.testing.assert_array_equal(gpu["meta"][t0:t1], ora["meta"], err_msg=f"{label}: meta")
    off = gpu["off"][c0:c1 + 1].astype(np.int64)
    np.testing.assert_array_equal(off - off[0], ora["off"].astype(np.int64), err_msg=f"{label}: chunk offsets")
    np.testing.assert_array_equal(gpu["payload"][off[0]:off[-1]], ora["payload"], err_msg=f"{label}: payload")
    np.testing.assert_array_equal(gpu["out"][t0 * tile:t1 * tile], ora["out"], err_msg=f"{label}: reconstruction")
    assert ora["status"] == ok_status and ora["dstatus"] == 0, (label, ora["status"], ora["dstatus"])
