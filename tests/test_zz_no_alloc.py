"""hq_encode_c_noalloc, the encode that allocates nothing (its workspace is
a static device array in the library), against hq_encode_c with a workspace
the caller allocates: bit-exact streams on two calls in a row, the second
with a smaller input, and a size past the static workspace rejected before
any device work."""
import ctypes

import numpy as np
import pytest
import torch

from hq_testutil import rate_c
from kv_cache_tile_amd import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from kv_cache_tile_amd import hq
    hq.lib()


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def _buffers(x2, tile, lat, c, kv, dev):
    p = hq.plan_c(hq.BF16, x2.shape[0], x2.shape[1], tile, lat, c, kv)
    return dict(payload=torch.zeros(p.payload_cap_words, dtype=torch.int32, device=dev),
                step=torch.zeros(p.tiles, dtype=torch.int16, device=dev),
                meta=torch.zeros(p.tiles, dtype=torch.int16, device=dev),
                off=torch.zeros(p.chunks + 1, dtype=torch.int32, device=dev),
                status=torch.zeros(1, dtype=torch.int32, device=dev))


def _host(b):
    torch.cuda.synchronize()
    w = int(b["off"][-1].item())
    return (b["step"].cpu().numpy(), b["meta"].cpu().numpy(), b["off"].cpu().numpy(),
            b["payload"][:w].cpu().numpy(), int(b["status"].item()))


def test_noalloc_matches_encode_c_twice():
    dev = _dev()
    L = hq.lib()
    cases = [("weights 4096x4096", workloads.gaussian_outlier_channels(4096, 4096, key=1), 128, 0, 4.0),
             ("KV 3000 x 128", workloads.gaussian(3000, 128, key=2), 128, 1, 2.0)]
    for label, x, tile, kv, bps in cases:
        xd = workloads.to_bf16(x).to(dev)
        c = rate_c("E8", tile, bps, kv)
        print(f"[case] no-alloc encode {label}", flush=True)
        ref = _buffers(xd, tile, "E8", c, kv, dev)
        ws = torch.zeros(hq.plan_c(hq.BF16, xd.shape[0], xd.shape[1], tile, "E8", c, kv).workspace_bytes,
                         dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        rc = L.hq_encode_c(xd.data_ptr(), hq.BF16, xd.shape[0], xd.shape[1], tile, 8, c, 7, kv,
                           ref["payload"].data_ptr(), ref["payload"].numel(), ref["step"].data_ptr(),
                           ref["meta"].data_ptr(), ref["off"].data_ptr(), ref["status"].data_ptr(), ws.data_ptr(),
                           ws.numel(), stream)
        assert rc == 0
        got = _buffers(xd, tile, "E8", c, kv, dev)
        rc = L.hq_encode_c_noalloc(xd.data_ptr(), hq.BF16, xd.shape[0], xd.shape[1], tile, 8, c, 7, kv,
                                   got["payload"].data_ptr(), got["payload"].numel(), got["step"].data_ptr(),
                                   got["meta"].data_ptr(), got["off"].data_ptr(), got["status"].data_ptr(), stream)
        assert rc == 0
        a, b = _host(ref), _host(got)
        for u, v in zip(a[:4], b[:4]):
            np.testing.assert_array_equal(u, v)
        assert a[4] == b[4] == 0


def test_noalloc_rejects_past_its_workspace():
    dev = _dev()
    L = hq.lib()
    t = torch.zeros(64, dtype=torch.int32, device=dev)
    c = rate_c("E8", 64, 4.0)
    rows = 64 * 130977                                    # 130977 chunks of 64 tiles of 64: one too many
    rc = L.hq_encode_c_noalloc(t.data_ptr(), hq.BF16, rows, 64, 64, 8, c, 0, 0, t.data_ptr(), 1 << 40,
                               t.data_ptr(), t.data_ptr(), t.data_ptr(), t.data_ptr(), None)
    assert rc == -3                                       # HQ_ENOSPC, nothing launched
    rows = 64 * 130976
    p = hq.plan_c(hq.BF16, rows, 64, 64, "E8", c)
    assert p.workspace_bytes == 1 << 20
