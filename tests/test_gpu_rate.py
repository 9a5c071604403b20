"""GPU parity of closed-loop rate control and of explicit rate constants
(gist.science explainer of HyperQuant, Methodology section 3: the realized
rate lands within about 0.01 bps of the target).  The library's bisection
(through the C ABI) must take the oracle's steps exactly: the same constant,
rate and number of encodes, and a bit-exact stream and reconstruction."""
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


def _inputs(kind, tile, kv, dtype, rows=256, cols=1024):
    x = workloads.gaussian(rows, cols, key=5) if kind == "gauss" else \
        workloads.student_t_outlier_cols(rows, cols, key=3, n_out=8)
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        xo = workloads.bf16_bits(t)
    else:
        xo = x
    if kv:
        t, xo = t.reshape(-1, tile), xo.reshape(-1, tile)
    return t.to(_dev()), xo


def _bits(t):
    return workloads.bf16_bits(t).reshape(-1) if t.dtype == torch.bfloat16 else t.cpu().numpy().view(np.uint32).reshape(-1)


def _check_stream(h, e, xo, tile, lat, c, seed, kv, dtype):
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h.step.cpu().numpy().view(np.uint16), e.step)
    np.testing.assert_array_equal(h.meta.cpu().numpy().view(np.uint16), e.meta)
    np.testing.assert_array_equal(h.chunk_off.cpu().numpy().view(np.uint32), e.chunk_off)
    words = h.payload_words()
    np.testing.assert_array_equal(h.payload[:words].cpu().numpy().view(np.uint32), e.payload)
    xh = hq.decode(h)
    torch.cuda.synchronize()
    rows, cols = xo.shape
    ref, st = oracle.decode(e, rows, cols, tile, lat, c, seed, oracle.BF16 if dtype == "bf16" else oracle.F32,
                            int(kv))
    assert st == oracle.OK and h.flags() == 0
    np.testing.assert_array_equal(_bits(xh), ref.reshape(-1).view(np.uint16 if dtype == "bf16" else np.uint32))


CASES = [("E8", 256, False, 4.0, "bf16"), ("D4", 128, False, 3.0, "bf16"), ("Z", 64, False, 5.0, "f32"),
         ("A2", 128, False, 3.25, "bf16"), ("E8", 128, True, 2.0, "bf16"), ("E8", 128, False, 3.3, "bf16")]


@pytest.mark.parametrize("kind", ["gauss", "student"])
@pytest.mark.parametrize("lat,tile,kv,R,dtype", CASES)
def test_rate_search_takes_the_oracles_steps(lat, tile, kv, R, dtype, kind):
    xd, xo = _inputs(kind, tile, kv, dtype)
    print(f"[case] rate search {lat} n={tile} kv={kv} R={R} {dtype} {kind}", flush=True)
    h = hq.encode_rate(xd, tile, lat, R, seed=9, kv=kv)
    c, r, n, e = oracle.rate_search(xo, tile, lat, R, 9, int(kv))
    assert (h.c, h.extra["rate"], h.extra["encodes"]) == (c, r, n)
    assert abs(r - float(np.float32(R))) <= 0.01
    _check_stream(h, e, xo, tile, lat, c, 9, kv, dtype)


@pytest.mark.parametrize("f", [0.37, 1.0, 2.9])
@pytest.mark.parametrize("lat,tile,kv", [("E8", 256, False), ("A2", 128, False), ("E8", 128, True)])
def test_explicit_constant(lat, tile, kv, f):
    # off-table constants: the step, the tile bound and the decoder's staging
    # follow c
    xd, xo = _inputs("student", tile, kv, "bf16", rows=130, cols=512)
    c = float(np.float32(rate_c(lat, tile, 2.0 if kv else 4.0, int(kv)) * f))
    print(f"[case] explicit c={c} {lat} n={tile} kv={kv}", flush=True)
    h = hq.encode_c(xd, tile, lat, c, seed=21, kv=kv)
    e = oracle.encode(xo, tile, lat, c, 21, int(kv))
    _check_stream(h, e, xo, tile, lat, c, 21, kv, "bf16")


def test_rate_search_llama_projection_full():
    # 4096 x 4096 bf16 (Gaussian weights with 1% outlier channels): the whole
    # search against the oracle's
    x = workloads.config_tensor(1)
    t = torch.from_numpy(x).to(torch.bfloat16)
    xo = workloads.bf16_bits(t)
    print("[case] rate search 4096x4096 E8 n=128 R=4", flush=True)
    h = hq.encode_rate(t.to(_dev()), 128, "E8", 4.0, seed=1)
    c, r, n, e = oracle.rate_search(xo, 128, "E8", 4.0, 1)
    assert (h.c, h.extra["rate"], h.extra["encodes"]) == (c, r, n)
    assert abs(r - 4.0) <= 0.01
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h.payload[:h.payload_words()].cpu().numpy().view(np.uint32), e.payload)


@pytest.mark.parametrize("kind", ["zeros", "nan_row"])
def test_rate_search_degenerate_inputs(kind):
    # an all-zero tensor cannot reach the target (every tile costs its coset
    # bits and one unary bit a symbol): the search runs down to the bracket's
    # end; a non-finite row is coded as zero and flagged.  Both sides take the
    # same steps either way.
    x = np.zeros((256, 512), np.float32) if kind == "zeros" else workloads.gaussian(256, 512, key=8)
    if kind == "nan_row":
        x[17, 100] = np.nan
    t = torch.from_numpy(x).to(torch.bfloat16)
    xo = workloads.bf16_bits(t)
    print(f"[case] rate search degenerate {kind}", flush=True)
    h = hq.encode_rate(t.to(_dev()), 128, "E8", 4.0, seed=3)
    c, r, n, e = oracle.rate_search(xo, 128, "E8", 4.0, 3)
    assert (h.c, h.extra["rate"], h.extra["encodes"]) == (c, r, n)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(h.payload[:h.payload_words()].cpu().numpy().view(np.uint32), e.payload)
    np.testing.assert_array_equal(h.step.cpu().numpy().view(np.uint16), e.step)
    if kind == "zeros":
        assert r < 1.2 and n > 5           # 144 bits per 128-scalar tile, far below the target
    else:
        assert h.flags() == hq.FLAG_NONFINITE and e.status == oracle.ENONFINITE


# The length pass (hq_encode_length_c): the payload word count the encoder
# would write, chunk_off[C], without writing a stream.  Ragged last chunks
# (130 x 768 scalars: 390 tiles at n = 256, 6 in the last chunk), every
# lattice, both dtypes, KV, off-table constants, and degenerate tiles.
LENGTH_CASES = [("E8", 256, False, "bf16", 4.0), ("E8", 128, True, "bf16", 2.0), ("D4", 64, False, "f32", 3.0),
                ("A2", 128, False, "bf16", 5.0), ("Z", 128, False, "bf16", 4.0), ("E8", 64, False, "f32", 6.0),
                ("A2", 64, True, "f32", 2.5)]


@pytest.mark.parametrize("f", [0.37, 1.0, 2.9])
@pytest.mark.parametrize("lat,tile,kv,dtype,R", LENGTH_CASES)
def test_length_pass_counts_the_encoders_words(lat, tile, kv, dtype, R, f):
    xd, xo = _inputs("student", tile, kv, dtype, rows=130, cols=768)
    c = float(np.float32(rate_c(lat, tile, R, int(kv)) * f))
    print(f"[case] length pass {lat} n={tile} kv={kv} {dtype} c={c}", flush=True)
    words = hq.encode_length_c(xd, tile, lat, c, seed=13, kv=kv)
    h = hq.encode_c(xd, tile, lat, c, seed=13, kv=kv)
    e = oracle.encode(xo, tile, lat, c, 13, int(kv))
    torch.cuda.synchronize()
    assert int(words.item()) == int(e.chunk_off[-1]) == h.payload_words()
    # a second pass adds to the same counter
    hq.encode_length_c(xd, tile, lat, c, seed=13, kv=kv, out=words)
    assert int(words.item()) == 2 * int(e.chunk_off[-1])


@pytest.mark.parametrize("kind", ["zeros", "nan_inf", "tiny_huge"])
def test_length_pass_degenerate_tiles(kind):
    x = workloads.gaussian(192, 1024, key=4)
    if kind == "zeros":
        x[:] = 0.0
    elif kind == "nan_inf":
        x[3, 10], x[77, 500], x[150, 0] = np.nan, np.inf, -np.inf     # non-finite tiles count as zero tiles
    else:
        x[:64] *= 1e-38
        x[64:128] *= 1e37
    t = torch.from_numpy(x).to(torch.bfloat16)
    xo = workloads.bf16_bits(t)
    c = rate_c("E8", 128, 4.0, 0)
    print(f"[case] length pass degenerate {kind}", flush=True)
    words = hq.encode_length_c(t.to(_dev()), 128, "E8", c, seed=2)
    e = oracle.encode(xo, 128, "E8", c, 2, 0)
    torch.cuda.synchronize()
    assert int(words.item()) == int(e.chunk_off[-1])


def test_length_pass_dit_layer():
    # one 4096 x 16384 bf16 layer at n = 256 (4096 chunks, several a
    # workgroup): the length pass against the encoder's own chunk_off[C]
    x = workloads.dit_layer_device(4096, 16384, 0, _dev())
    c = rate_c("E8", 256, 4.0, 0)
    print("[case] length pass 4096x16384 E8 n=256", flush=True)
    words = hq.encode_length_c(x, 256, "E8", c, seed=5)
    h = hq.encode_c(x, 256, "E8", c, seed=5)
    torch.cuda.synchronize()
    assert int(words.item()) == h.payload_words()
