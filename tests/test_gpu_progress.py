"""Forward progress of the encode (the chunk-offset look-back).

A look-back waits only for groups of chunks taken before its own, by
workgroups already running, so an encode completes however few of its
workgroups are resident at once: a grid several times larger than fits the
device gives the same stream as the default grid.  The wait is bounded: with
the bound forced to zero polls from the host every workgroup still ends, the
status is clean or HQ_FLAG_STALL, and the workspace is left ready for the
next call."""
import numpy as np
import pytest
import torch

from kv_cache_tile_amd import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from kv_cache_tile_amd import hq
    hq.lib()


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def _stream_of(h):
    torch.cuda.synchronize()
    w = h.payload_words()
    return (h.step.cpu().numpy().copy(), h.meta.cpu().numpy().copy(), h.chunk_off.cpu().numpy().copy(),
            h.payload[:w].cpu().numpy().copy(), h.flags())


def _same(a, b):
    for u, v in zip(a[:4], b[:4]):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("tile,grid", [(256, 2048), (128, 2048)])
def test_oversubscribed_grid(tile, grid, monkeypatch):
    # one chunk per group and a grid of 2048 workgroups (the most the
    # library launches), 4x (n = 256: 2 workgroups per CU) or 2x (n = 128: 4
    # per CU) what the device holds at once: many workgroups start only after
    # others have left
    dev = _dev()
    T = 64 * grid + 64 * 7 + 5
    x = workloads.to_bf16(workloads.gaussian(T, tile, key=tile + 5)).to(dev)
    print(f"[case] oversubscribed grid={grid} tile={tile} T={T}", flush=True)
    ref = _stream_of(hq.encode(x, tile, "E8", 4.0, 77))
    assert ref[4] == 0
    monkeypatch.setenv("HQ_ENCODE_GROUP_CHUNKS", "1")
    monkeypatch.setenv("HQ_ENCODE_GRID", str(grid))
    for _ in range(2):
        got = _stream_of(hq.encode(x, tile, "E8", 4.0, 77))
        assert got[4] == 0
        _same(got, ref)
    monkeypatch.delenv("HQ_ENCODE_GRID")
    monkeypatch.delenv("HQ_ENCODE_GROUP_CHUNKS")
    _same(_stream_of(hq.encode(x, tile, "E8", 4.0, 77)), ref)


@pytest.mark.parametrize("tile", [128, 256])
def test_bounded_wait_forced(tile, monkeypatch):
    # zero polls: a look-back that finds a predecessor unpublished gives up at
    # once; the kernel still ends and flags it, and a normal encode on the
    # same workspace afterwards is exact
    dev = _dev()
    T = 64 * 3000 + 9
    x = workloads.to_bf16(workloads.gaussian(T, tile, key=tile + 9)).to(dev)
    print(f"[case] forced bounded wait tile={tile} T={T}", flush=True)
    ref = _stream_of(hq.encode(x, tile, "E8", 4.0, 5))
    assert ref[4] == 0
    monkeypatch.setenv("HQ_ENCODE_SPIN_LIMIT", "0")
    for grid in ("0", "1500"):
        if grid != "0":
            monkeypatch.setenv("HQ_ENCODE_GRID", grid)
            monkeypatch.setenv("HQ_ENCODE_GROUP_CHUNKS", "2")
        got = _stream_of(hq.encode(x, tile, "E8", 4.0, 5))
        assert got[4] in (0, hq.FLAG_STALL)
        if got[4] == 0:
            _same(got, ref)
    monkeypatch.delenv("HQ_ENCODE_SPIN_LIMIT")
    monkeypatch.delenv("HQ_ENCODE_GRID")
    monkeypatch.delenv("HQ_ENCODE_GROUP_CHUNKS")
    _same(_stream_of(hq.encode(x, tile, "E8", 4.0, 5)), ref)
