"""GPU parity of the int8 product path (gist.science explainer of HyperQuant,
Key Contributions, "Hardware Integration"; Methodology section 2): codes 2P
from the decoder, the activations' int8 RHT, and the matrix-core product,
each bit-exact against the oracle; and the product read straight from the
stream in one launch (hq_codes_matmul_fused; "Significance and Claims":
decoding fused with the product), bit-exact against the same oracle chain."""
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
    xd = torch.from_numpy(x).to(dev)
    y = hq.matmul_compressed(h, xd)                           # (the fused product: rows are whole chunks)
    qd, scd = hq.act_quant(xd, 256, seed)
    y2 = hq.codes_matmul(hq.decode_codes(h), h.step, 256, qd, scd)   # the two-pass path
    torch.cuda.synchronize()
    c = rate_c("E8", 256, 4.0)
    e = oracle.encode(wo, 256, "E8", c, seed)
    codes, st, flag = oracle.decode_codes(e, 4096, 16384, 256, "E8", c, seed)
    q, sc = oracle.act_quant(x, 256, seed)
    ref = oracle.codes_matmul(codes, e.step, 256, q, sc)
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    np.testing.assert_array_equal(y2.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert flag == 0 and h.flags() == 0


def _nan_equal(a, b):
    a, b = np.asarray(a), np.asarray(b)
    both_nan = np.isnan(a) & np.isnan(b)
    np.testing.assert_array_equal(np.where(both_nan, 0, a).view(np.uint32), np.where(both_nan, 0, b).view(np.uint32))


def test_act_quant_non_finite():
    dev = _dev()
    x = workloads.gaussian(3, 512, key=6)
    x[0, 5] = np.nan
    x[1, 300] = np.inf
    x[2, 0] = -np.inf
    q, sc = hq.act_quant(torch.from_numpy(x).to(dev), 128, 4)
    rq, rsc = oracle.act_quant(x, 128, 4)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    _nan_equal(sc.cpu().numpy(), rsc)


@pytest.mark.parametrize("lat,tile,bps", [("E8", 256, 4.0), ("E8", 128, 3.0), ("D4", 128, 4.0), ("Z", 64, 5.0),
                                          ("E8", 64, 8.0)])
def test_fused_product(lat, tile, bps):
    # rows not a multiple of 8, two chunks a row, activations in two blocks of 32
    rows, batch = 43, 37
    cols = 2 * 64 * tile
    print(f"[case] fused product {lat} n={tile} bps={bps} rows={rows} batch={batch}", flush=True)
    h, e = _weights(lat, tile, rows, cols, bps, key=tile)
    x = workloads.gaussian(batch, cols, key=rows + tile)
    q, sc = hq.act_quant(torch.from_numpy(x).to(_dev()), tile, 7)
    qb, scb = hq.act_quant(torch.from_numpy(x).to(_dev()), tile, 7, blocked=True)
    status = torch.zeros(1, dtype=torch.int32, device=_dev())
    y = hq.codes_matmul_fused(h, qb, scb, status)
    torch.cuda.synchronize()
    c = rate_c(lat, tile, bps)
    codes, st, flag = oracle.decode_codes(e, rows, cols, tile, lat, c, 7)
    ref = oracle.codes_matmul(codes, e.step, tile, q.cpu().numpy(), sc.cpu().numpy())
    np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))
    assert int(status.item()) == (hq.FLAG_RANGE if flag else 0)


def _unblock(qb, batch, cols, tile):
    # the blocked order [batch / 32][tile t][32-code step k][activation % 32][32]
    # back to [batch][cols]
    nb = (batch + 31) // 32
    a = qb.reshape(nb, cols // tile, tile // 32, 32, 32).permute(0, 3, 1, 2, 4).reshape(nb * 32, cols)
    return a[:batch]


@pytest.mark.parametrize("tile,batch", [(64, 37), (128, 64), (256, 5), (256, 33)])
def test_act_quant_blocked(tile, batch):
    # the same codes and scales as hq_act_quant, in the matrix-core order
    cols = 3 * tile
    x = torch.from_numpy(workloads.gaussian(batch, cols, key=tile + batch)).to(_dev())
    q, sc = hq.act_quant(x, tile, 5)
    qb, scb = hq.act_quant(x, tile, 5, blocked=True)
    torch.cuda.synchronize()
    assert qb.numel() == (batch + 31) // 32 * 32 * cols
    assert torch.equal(_unblock(qb.cpu(), batch, cols, tile), q.cpu())
    assert torch.equal(scb.cpu(), sc.cpu())
    with pytest.raises(hq.HQError, match="blocked=True"):
        hq.codes_matmul_fused(hq.encode(torch.zeros(8, 64 * tile, device=_dev()), tile, "E8", 4.0, 1),
                              q, sc, torch.zeros(1, dtype=torch.int32, device=_dev()))


def test_fused_product_non_finite_activations():
    # a NaN or an infinity in an activation tile makes that tile's scale
    # non-finite: its products are NaN in the fused chain as in the oracle's,
    # and the other activations' outputs are untouched; 70 activations (three
    # blocks of 32, the last partial)
    dev = _dev()
    lat, tile, rows, batch = "E8", 128, 24, 70
    cols = 64 * tile
    h, e = _weights(lat, tile, rows, cols, 4.0, key=21)
    x = workloads.gaussian(batch, cols, key=22)
    x[3, 17] = np.nan
    x[40, 5000] = np.inf
    x[69, 1] = -np.inf
    xt = torch.from_numpy(x).to(dev)
    q, sc = hq.act_quant(xt, tile, 7)
    qb, scb = hq.act_quant(xt, tile, 7, blocked=True)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    y = hq.codes_matmul_fused(h, qb, scb, status)
    torch.cuda.synchronize()
    c = rate_c(lat, tile, 4.0)
    codes, st, flag = oracle.decode_codes(e, rows, cols, tile, lat, c, 7)
    ref = oracle.codes_matmul(codes, e.step, tile, q.cpu().numpy(), sc.cpu().numpy())
    _nan_equal(y.cpu().numpy(), ref)
    assert np.isnan(ref[3]).all() and np.isfinite(ref[4]).all()


def test_fused_product_corrupt_streams():
    # corrupt tiles and chunks give zero codes (and the flag) on both sides;
    # a non-finite step makes that tile's products NaN on both sides
    dev = _dev()
    lat, tile, rows, cols, batch = "E8", 128, 16, 2 * 64 * 128, 8
    h, e = _weights(lat, tile, rows, cols, 4.0, key=11)
    x = workloads.gaussian(batch, cols, key=12)
    q, sc = hq.act_quant(torch.from_numpy(x).to(dev), tile, 7)
    qb, scb = hq.act_quant(torch.from_numpy(x).to(dev), tile, 7, blocked=True)
    c = rate_c(lat, tile, 4.0)
    rng = np.random.default_rng(3)
    for trial in range(6):
        pay, meta, off, step = e.payload.copy(), e.meta.copy(), e.chunk_off.copy(), e.step.copy()
        if trial % 3 == 0:
            for _ in range(2):
                w_ = rng.integers(0, pay.size)
                pay[w_] ^= np.uint32(1) << np.uint32(rng.integers(0, 32))
        elif trial % 3 == 1:
            meta[rng.integers(0, meta.size)] += np.uint16(8)
        else:
            step[rng.integers(0, step.size)] = 0x7F80
        hh = hq.HQTensor(torch.from_numpy(pay.view(np.int32)).to(dev), torch.from_numpy(step.view(np.int16)).to(dev),
                         torch.from_numpy(meta.view(np.int16)).to(dev), torch.from_numpy(off.view(np.int32)).to(dev),
                         torch.zeros(1, dtype=torch.int32, device=dev), (rows, cols), torch.bfloat16, tile, lat, 4.0, 7)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        y = hq.codes_matmul_fused(hh, qb, scb, status)
        torch.cuda.synchronize()
        ee = oracle.Encoded(step, meta, off, pay, 0)
        codes, st, flag = oracle.decode_codes(ee, rows, cols, tile, lat, c, 7)
        ref = oracle.codes_matmul(codes, step, tile, q.cpu().numpy(), sc.cpu().numpy())
        _nan_equal(y.cpu().numpy(), ref)
        assert bool(int(status.item()) & hq.FLAG_CORRUPT) == (st == oracle.ECORRUPT)


def test_matmul_compressed_raises_on_saturation():
    # at 8 bps some codes pass 127: the product is not x W_hat^T and the
    # binding says so, with a status word of its own
    dev = _dev()
    h, e = _weights("E8", 64, 16, 64 * 64, 8.0, key=13)
    x = torch.from_numpy(workloads.gaussian(4, 64 * 64, key=14)).to(dev)
    with pytest.raises(hq.HQError, match="saturated"):
        hq.matmul_compressed(h, x)
    assert h.flags() == 0
