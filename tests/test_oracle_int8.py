"""Pins of the oracle's int8 product path (gist.science explainer of
HyperQuant, Key Contributions, "Hardware Integration": int8 matrix-core paths
on the post-RHT lattice output; Methodology section 2: the lattice's integer
embedding).  The codes must rebuild the codec's own decode exactly; the
activation quantization must stay within half a step; the product's integer
part must be exact and its result must approximate W_hat x within the
activation quantization bound."""
import numpy as np
import pytest

import oracle
from hq_testutil import rate_c
from kv_cache_tile_amd import workloads


def _stream(lat, tile, rows=96, cols=1024, bps=4.0, seed=7):
    w = workloads.gaussian(rows, cols, key=3)
    c = rate_c(lat, tile, bps)
    e = oracle.encode(w, tile, lat, c, seed)
    return w, e, c


@pytest.mark.parametrize("lat,tile", [("E8", 256), ("E8", 128), ("D4", 128), ("Z", 64)])
def test_codes_rebuild_the_decode_exactly(lat, tile):
    w, e, c = _stream(lat, tile)
    rows, cols = w.shape
    codes, st, flag = oracle.decode_codes(e, rows, cols, tile, lat, c, 7)
    assert st == oracle.OK and flag == 0
    xh, st2 = oracle.decode(e, rows, cols, tile, lat, c, 7, oracle.F32)
    s = (e.step.astype(np.uint32) << 16).view(np.float32)
    v = (codes.reshape(-1, tile).astype(np.float32) * np.float32(0.5)) * s[:, None]
    ref = np.stack([oracle.rht_inverse(vt, 7) for vt in v]).reshape(rows, cols)
    np.testing.assert_array_equal(ref.view(np.uint32), xh.view(np.uint32))


def test_codes_reject_dither_and_a2_and_flag_saturation():
    w, e, c = _stream("A2", 128)
    assert oracle.decode_codes(e, *w.shape, 128, "A2", c, 7)[1] == oracle.EINVAL
    # a high rate puts codes beyond 127 (|2P| grows as the step shrinks)
    w2, e2, c2 = _stream("E8", 256, bps=8.0)
    codes, st, flag = oracle.decode_codes(e2, *w2.shape, 256, "E8", c2, 7)
    assert flag == 1 and np.abs(codes.astype(int)).max() == 127


def test_activation_quantization_within_half_a_step():
    x = workloads.gaussian(4, 1024, key=9)
    q, sc = oracle.act_quant(x, 256, 11)
    for b in range(4):
        for t in range(4):
            y = oracle.rht_forward(x[b, 256 * t:256 * (t + 1)], 11).astype(np.float64)
            a = float(sc[b, t])
            assert a == pytest.approx(np.abs(y).max() / 127, rel=1e-6)
            assert np.abs(y - a * q[b, 256 * t:256 * (t + 1)]).max() <= a / 2 * (1 + 1e-5)
            assert np.abs(q[b, 256 * t:256 * (t + 1)].astype(int)).max() == 127


def test_product_integer_part_and_end_to_end_bound():
    lat, tile = "E8", 256
    w, e, c = _stream(lat, tile, rows=64, cols=1024)
    rows, cols = w.shape
    codes, _, _ = oracle.decode_codes(e, rows, cols, tile, lat, c, 7)
    x = workloads.gaussian(3, cols, key=21)
    q, sc = oracle.act_quant(x, tile, 7)
    y = oracle.codes_matmul(codes, e.step, tile, q, sc).astype(np.float64)
    s = (e.step.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(rows, cols // tile)
    # exact integer dot products, then the scaled sum in fp64
    I = np.einsum("rtk,btk->brt", codes.reshape(rows, -1, tile).astype(np.int64), q.reshape(3, -1, tile).astype(np.int64))
    y64 = 0.5 * (I * (s[None] * sc.astype(np.float64)[:, None, :])).sum(-1)
    tiles = cols // tile
    assert np.all(np.abs(y - y64) <= tiles * 2.0 ** -23 * 0.5 * np.abs(I * (s[None] * sc[:, None, :])).sum(-1) + 1e-30)
    # against W_hat x with W_hat the codec's own decode: the only error left is
    # the activation's int8 quantization, |x' - a q| <= a / 2 per coordinate
    xh, _ = oracle.decode(e, rows, cols, tile, lat, c, 7, oracle.F32)
    ref = x.astype(np.float64) @ xh.astype(np.float64).T
    bound = 0.5 * (np.abs(codes.reshape(rows, -1, tile)).sum(-1)[None] * s[None] * sc.astype(np.float64)[:, None, :] / 2).sum(-1)
    assert np.all(np.abs(y - ref) <= bound * 1.01 + 1e-6)


def test_act_quant_non_finite_tiles():
    # a NaN or an infinity makes the tile's scale non-finite and its codes 0
    # (the product over the tile is then NaN); the other tiles are untouched
    x = workloads.gaussian(3, 512, key=5)
    ref_q, ref_a = oracle.act_quant(x, 128, 4)
    x[0, 5] = np.nan
    x[1, 300] = np.inf
    q, a = oracle.act_quant(x, 128, 4)
    assert np.isnan(a[0, 0]) and np.isinf(a[1, 2])
    assert not q[0, :128].any() and not q[1, 256:384].any()
    keep = np.ones_like(a, bool)
    keep[0, 0] = keep[1, 2] = False
    np.testing.assert_array_equal(a[keep], ref_a[keep])
    qm = np.ones_like(q, bool)
    qm[0, :128] = qm[1, 256:384] = False
    np.testing.assert_array_equal(q[qm], ref_q[qm])
    codes = np.ones((2, 512), np.int8)
    y = oracle.codes_matmul(codes, np.full(8, 0x3F80, np.uint16), 128, q, a)
    assert np.all(np.isnan(y[:2]))
