"""GPU parity of the int8 product path (gist.science explainer of HyperQuant,
Key Contributions, "Hardware Integration"; Methodology section 2): codes 2P
from the decoder, the activations' int8 RHT, and the matrix-core product,
each bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from hq_testutil import rate_c
from kv_cache_tile_amd import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from kv_cache_tile_amd import hq
    hq.lib()                        # no fallback: a missing library fails every test


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def _weights(lat, tile, rows, cols, bps=4.0, seed=7, key=3):
    w = workloads.gaussian(rows, cols, key=key)
    wt = torch.from_numpy(w).to(torch.bfloat16)
    wo = workloads.bf16_bits(wt)
    h = hq.encode(wt.to(_dev()), tile, lat, bps, seed)
    e = oracle.encode(wo, tile, lat, rate_c(lat, tile, bps), seed)
    return h, e


@pytest.mark.parametrize("lat,tile,bps", [("E8", 256, 4.0), ("E8", 128, 3.0), ("D4", 128, 4.0), ("Z", 64, 5.0),
                                          ("E8", 256, 8.0)])
def test_decode_codes(lat, tile, bps):
    rows, cols = 67, 1024
    print(f"[case] decode codes {lat} n={tile} bps={bps}", flush=True)
    h, e = _weights(lat, tile, rows, cols, bps)
    codes = hq.decode_codes(h)
    torch.cuda.synchronize()
    ref, st, flag = oracle.decode_codes(e, rows, cols, tile, lat, rate_c(lat, tile, bps), 7)
    assert st == oracle.OK
    np.testing.assert_array_equal(codes.cpu().numpy(), ref)
    assert h.flags() == (hq.FLAG_RANGE if flag else 0)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("tile", [64, 128, 256])
def test_act_quant(tile, dt):
    x = workloads.gaussian(5, 1024, key=tile)
    x[2, :tile] = 0.0                               # a zero tile: scale 0, codes 0
    xt = torch.from_numpy(x)
    if dt == "bf16":
        xt = xt.to(torch.bfloat16)
        xo = (workloads.bf16_bits(xt).astype(np.uint32) << 16).view(np.float32)
    else:
        xo = x
    print(f"[case] act quant n={tile} {dt}", flush=True)
    q, sc = hq.act_quant(xt.to(_dev()), tile, 11)
    rq, rsc = oracle.act_quant(xo, tile, 11)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), rsc.view(np.uint32))


@pytest.mark.parametrize("rows,batch,tile", [(100, 37, 256), (32, 1, 128), (64, 64, 64), (7, 3, 256)])
def test_codes_matmul(rows, batch, tile):
    cols = 4 * tile
    print(f"[case] codes matmul rows={rows} batch={batch} n={tile}", flush=True)
    h, e = _weights("E8", tile, rows, cols)
    codes = hq.decode_codes(h)
    x = torch.from_numpy(workloads.gaussian(batch, cols, key=rows)).to(_dev())
    q, sc = hq.act_quant(x, tile, 7)
    y = hq.codes_matmul(codes, h.step, tile, q, sc)
    torch.cuda.synchronize()
    ref = oracle.codes_matmul(codes.cpu().numpy(), h.step.cpu().numpy().view(np.uint16), tile, q.cpu().numpy(),
                              sc.cpu().numpy())
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_dit_layer_product_full():
    # one 4096 x 16384 bf16 DiT layer (E8, 4 bps, n = 256) times 32 activations,
    # the whole chain against the oracle's
    dev = _dev()
    w = workloads.dit_layer(4096, 16384, key=4, layer=0)
    wt = torch.from_numpy(w).to(torch.bfloat16)
    wo = workloads.bf16_bits(wt)
    seed = workloads.codec_seed(4, 0)
    print("[case] int8 product DiT layer x 32", flush=True)
    h = hq.encode(wt.to(dev), 256, "E8", 4.0, seed)
    x = workloads.gaussian(32, 16384, key=77)
    y = hq.matmul_compressed(h, torch.from_numpy(x).to(dev))
    torch.cuda.synchronize()
    c = rate_c("E8", 256, 4.0)
    e = oracle.encode(wo, 256, "E8", c, seed)
    codes, st, flag = oracle.decode_codes(e, 4096, 16384, 256, "E8", c, seed)
    q, sc = oracle.act_quant(x, 256, seed)
    ref = oracle.codes_matmul(codes, e.step, 256, q, sc)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert h.flags() == (hq.FLAG_RANGE if flag else 0)
