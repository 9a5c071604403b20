"""The sliced oracle that the full-size parity tests run in parallel host
processes: chunk-aligned slices of tiles, encoded and decoded as tensors of
their own (the dither indexed by the global coordinate through tile_base),
give exactly the whole tensor's stream and reconstruction."""
import numpy as np
import pytest

import oracle
import oracle_pool
from hq_testutil import rate_c
from kv_cache_tile_amd import workloads


def _whole(x, tile, lat, c, seed, dither):
    e = oracle.encode(x, tile, lat, c, seed, dither)
    dt = oracle.F32 if x.dtype == np.float32 else oracle.BF16
    xh, st = oracle.decode(e, x.shape[0], x.shape[1], tile, lat, c, seed, dt, dither)
    assert st == oracle.OK
    bits = xh.view(np.uint32) if xh.dtype == np.float32 else xh.view(np.uint16)
    return dict(step=e.step, meta=e.meta, off=e.chunk_off, payload=e.payload, out=bits.reshape(-1)), e.status


@pytest.mark.parametrize("lat,tile,dither", [("E8", 128, 0), ("E8", 128, 1), ("A2", 64, 1), ("D4", 256, 0),
                                             ("Z", 64, 1)])
def test_slices_reassemble_the_whole(lat, tile, dither):
    T = 64 * 9 + 13
    x = workloads.bf16_bits(workloads.to_bf16(workloads.gaussian(T, tile, key=tile + dither)))
    c = rate_c(lat, tile, 2.0 if dither else 4.0, dither)
    whole, st = _whole(x, tile, lat, c, 21, dither)
    for parts in (1, 3, 4, 10):
        for t0, t1 in oracle_pool.chunk_slices(T, parts):
            r = oracle_pool.oracle_slice((("array", x[t0:t1]), tile, lat, c, 21, dither, t0, False))
            oracle_pool.compare_slice(whole, t0, t1, tile, r, st, f"{lat} slice {t0}:{t1}")


def test_slice_with_wrong_base_differs():
    # the dither really is indexed by the global coordinate
    T = 64 * 3
    x = workloads.bf16_bits(workloads.to_bf16(workloads.gaussian(T, 128, key=3)))
    c = rate_c("E8", 128, 2.0, 1)
    whole, _ = _whole(x, 128, "E8", c, 5, 1)
    r = oracle_pool.oracle_slice((("array", x[64:128]), 128, "E8", c, 5, 1, 0, False))
    assert not np.array_equal(r["out"], whole["out"][64 * 128:128 * 128])


def test_spawned_pool_matches_in_process():
    # the same slices through spawned worker processes
    T = 64 * 5 + 3
    x = workloads.bf16_bits(workloads.to_bf16(workloads.gaussian(T, 128, key=9)))
    c = rate_c("E8", 128, 2.0, 1)
    tasks = [(("array", x[t0:t1]), 128, "E8", c, 2, 1, t0, True) for t0, t1 in oracle_pool.chunk_slices(T, 3)]
    pool = oracle_pool.make_pool(2)
    try:
        got = pool.map(oracle_pool.oracle_slice, tasks)
    finally:
        pool.close()
        pool.join()
    for task, r in zip(tasks, got):
        ref = oracle_pool.oracle_slice(task)
        for k in ("step", "meta", "off", "payload", "out", "x"):
            np.testing.assert_array_equal(r[k], ref[k])
