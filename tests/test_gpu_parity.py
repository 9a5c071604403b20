"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bit-exact on every integer/byte output (step, meta, chunk offsets,
payload words) and on the reconstruction (fp32 or bf16 bits).  Small cases
span several chunks and a ragged tail; the two smaller benchmark
configurations are checked whole here, the larger ones chunk by chunk on a
pool of oracle processes in test_gpu_full_parity."""
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


def to_device(x_np, dtype):
    """numpy fp32 -> device tensor of dtype; also returns the oracle's input
    (fp32 array, or bf16 bit patterns as uint16)."""
    t = torch.from_numpy(np.ascontiguousarray(x_np, np.float32))
    if dtype == "bf16":
        tb = t.to(torch.bfloat16)
        return tb.to(_dev()), workloads.bf16_bits(tb)
    return t.to(_dev()), np.ascontiguousarray(x_np, np.float32)


def gpu_encode(xd, tile, lat, bps, seed, kv):
    h = hq.kv_encode(xd, lat, bps, seed) if kv else hq.encode(xd, tile, lat, bps, seed)
    torch.cuda.synchronize()
    words = h.payload_words()
    return h, dict(step=h.step.cpu().numpy().view(np.uint16), meta=h.meta.cpu().numpy().view(np.uint16),
                   off=h.chunk_off.cpu().numpy().view(np.uint32),
                   payload=h.payload[:words].cpu().numpy().view(np.uint32), status=h.flags())


def out_bits(t):
    if t.dtype == torch.bfloat16:
        return workloads.bf16_bits(t)
    return t.cpu().numpy().view(np.uint32)


def oracle_out_bits(a):
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def check_full(x_np, tile, lat, bps, seed, kv, dtype):
    xd, xo = to_device(x_np, dtype)
    xd = xd.reshape(-1, tile) if kv else xd
    print(f"[case] full parity shape={tuple(x_np.shape)} tile={tile} {lat} bps={bps} kv={kv} {dtype}", flush=True)
    h, g = gpu_encode(xd, tile, lat, bps, seed, kv)
    c = rate_c(lat, tile, bps, int(kv))
    e = oracle.encode(xo.reshape(-1, x_np.shape[-1]) if not kv else xo.reshape(-1, tile), tile, lat, c, seed,
                      int(kv))
    np.testing.assert_array_equal(g["step"], e.step)
    np.testing.assert_array_equal(g["meta"], e.meta)
    np.testing.assert_array_equal(g["off"], e.chunk_off)
    np.testing.assert_array_equal(g["payload"], e.payload)
    assert g["status"] == (hq.FLAG_NONFINITE if e.status == oracle.ENONFINITE else 0)
    # decode of the GPU stream vs decode of the oracle stream
    xh = hq.decode(h)
    torch.cuda.synchronize()
    rows, cols = (xo.size // tile, tile) if kv else xo.shape
    ref, st = oracle.decode(e, rows, cols, tile, lat, c, seed,
                            oracle.BF16 if dtype == "bf16" else oracle.F32, int(kv))
    assert st == oracle.OK and h.flags() == g["status"]
    np.testing.assert_array_equal(out_bits(xh).reshape(-1), oracle_out_bits(ref).reshape(-1))
    return h, e


# ---------------------------------------------------------------- small cases
@pytest.mark.parametrize("kv", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tile", [64, 128, 256])
@pytest.mark.parametrize("lat", ["Z", "A2", "D4", "E8"])
def test_small_parity(lat, tile, dtype, kv):
    T = 200                                          # 3 full chunks + a ragged 8-tile chunk
    x = workloads.student_t_outlier_cols(T // 2, 2 * tile, key=tile + len(lat), n_out=2)
    check_full(x, tile, lat, 2.0 if kv else 4.0, seed=1000 + tile, kv=kv, dtype=dtype)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 129])
def test_tile_counts(T):
    x = workloads.gaussian(T, 128, key=T)
    check_full(x, 128, "E8", 4.0, seed=T, kv=False, dtype="bf16")


# The encoder stages several chunks per ticket (at most 4, and no more than
# LDS allows): chunk counts of 5, 6, 8, 10 and 17 give partial last groups and
# several groups, at both tile sizes the configurations use.  With the full
# grid every workgroup gets about one group; a grid capped at 2 or 3
# workgroups gives each several, alternating between the two halves of its
# staging area, with a group placed while the next one is in progress.
#
# The library picks the group size that shortens the busiest workgroup's
# sequence of chunks (with the full grid these inputs get groups of one
# chunk); a fixed size of 4 keeps the largest groups covered as well.
@pytest.mark.parametrize("grid_cap,group", [(0, 0), (2, 0), (3, 0), (0, 4), (2, 4), (3, 4)])
@pytest.mark.parametrize("chunks", [5, 6, 8, 10, 17])
@pytest.mark.parametrize("tile", [128, 256])
def test_chunk_groups(chunks, tile, grid_cap, group, monkeypatch):
    if grid_cap:
        monkeypatch.setenv("HQ_ENCODE_GRID_CAP", str(grid_cap))
    if group:
        monkeypatch.setenv("HQ_ENCODE_GROUP_CHUNKS", str(group))
    T = 64 * (chunks - 1) + 7
    x = workloads.gaussian(T, tile, key=1000 + chunks)
    check_full(x, tile, "E8", 4.0, seed=chunks, kv=False, dtype="bf16")


# The decoder streams a unit's words into LDS 16 bytes a lane; the stream's
# last vector, when it runs past payload_words, is read word by word.  An
# exact-size payload (a fresh copy of the valid words) reaches that path; tile
# counts here give every residue of the word count mod 4.
@pytest.mark.parametrize("tile", [128, 256])
@pytest.mark.parametrize("T", [37, 64, 65, 100, 127, 129, 191, 250])
def test_exact_size_payload(T, tile):
    x = workloads.gaussian(T, tile, key=3000 + T)
    xd, xo = to_device(x, "bf16")
    print(f"[case] exact-size payload T={T} tile={tile}", flush=True)
    h, g = gpu_encode(xd, tile, "E8", 4.0, T, False)
    words = g["payload"].size
    exact = torch.empty(words, dtype=torch.int32, device=_dev())
    exact.copy_(h.payload[:words])
    h2 = hq.HQTensor(exact, h.step, h.meta, h.chunk_off, torch.zeros_like(h.status), h.shape, h.dtype, h.tile,
                     h.lattice, h.bps, h.seed, h.kv)
    a, b = hq.decode(h), hq.decode(h2)
    torch.cuda.synchronize()
    assert h2.flags() == 0 and h.flags() == 0
    np.testing.assert_array_equal(out_bits(a), out_bits(b))
    c = rate_c("E8", tile, 4.0)
    e = oracle.encode(xo, tile, "E8", c, T)
    np.testing.assert_array_equal(g["payload"], e.payload)
    ref, st = oracle.decode(e, T, tile, tile, "E8", c, T, oracle.BF16)
    assert st == oracle.OK
    np.testing.assert_array_equal(out_bits(b).reshape(-1), oracle_out_bits(ref).reshape(-1))


@pytest.mark.parametrize("bps", [1.5, 3.0, 5.0, 8.0])
@pytest.mark.parametrize("tile", [128, 256])
def test_rate_extremes(bps, tile):
    x = workloads.gaussian(96, 2 * tile, key=int(bps * 4))
    check_full(x, tile, "E8", bps, seed=7, kv=False, dtype="f32")


def test_special_values():
    n = 128
    x = workloads.gaussian(40, 2 * n, key=9)
    x[0] = 0.0                                       # zero tiles
    x[1, :n] = 5.0                                   # constant tile
    x[2, 3] = np.nan                                 # non-finite tiles -> flagged, coded as zero
    x[3, 200] = np.inf
    x[4] = 1e-40                                     # subnormal inputs: step rounds to 0
    x[5] *= 1e30                                     # huge range
    x[6, :n] = 0.0; x[6, 7] = 1e3                    # one spike
    x[7] = np.float32(1.5e-45) * np.arange(2 * n)    # denormal ramp
    h, e = check_full(x, n, "E8", 4.0, seed=3, kv=False, dtype="f32")
    assert h.flags() == hq.FLAG_NONFINITE


@pytest.mark.parametrize("lat,n,kv", [("E8", 128, False), ("E8", 256, False), ("E8", 128, True), ("E8", 64, True),
                                      ("A2", 256, False), ("Z", 64, False), ("D4", 256, True), ("A2", 128, True)])
@pytest.mark.parametrize("odt", ["f32", "bf16"])
def test_decoder_step_rules(lat, n, kv, odt):
    # Steps the encoder never writes (negative, -0, subnormal, below 2^-124)
    # mark their tile corrupt; a +0 step over nonzero codes decodes to the
    # butterfly's signed zeros; the smallest valid steps decode exactly.  Bit
    # for bit against the oracle on the same stream.
    _dev()
    T, seed, bps = 150, 6, (2.0 if kv else 4.0)
    print(f"[case] step rules {lat} n={n} kv={kv} out={odt}", flush=True)
    x = workloads.gaussian(T, n, key=31)
    c = rate_c(lat, n, bps, int(kv))
    e = oracle.encode(x, n, lat, c, seed, dither=int(kv))
    step = e.step.copy()
    for t, v in {3: 0x0000, 10: 0x0180, 11: 0x01A5, 20: 0x017F, 30: 0x8000, 40: 0xC000, 50: 0x0001,
                 64: 0x0000, 70: 0x0200, 149: 0x0000}.items():
        step[t] = v
    ee = oracle.Encoded(step, e.meta, e.chunk_off, e.payload, 0)
    ref, st = oracle.decode(ee, T, n, n, lat, c, seed, oracle.F32 if odt == "f32" else oracle.BF16,
                            dither=int(kv))
    assert st == oracle.ECORRUPT
    pay = e.payload.astype(np.uint32)
    h = hq.HQTensor(torch.from_numpy(pay.view(np.int32)).to(_dev()),
                    torch.from_numpy(step.view(np.int16)).to(_dev()),
                    torch.from_numpy(e.meta.view(np.int16)).to(_dev()),
                    torch.from_numpy(e.chunk_off.view(np.int32)).to(_dev()),
                    torch.zeros(1, dtype=torch.int32, device=_dev()), (T, n),
                    torch.float32 if odt == "f32" else torch.bfloat16, n, lat, bps, seed, kv)
    out = hq.decode(h)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out_bits(out).reshape(-1), oracle_out_bits(ref).reshape(-1))
    assert h.flags() == hq.FLAG_CORRUPT


@pytest.mark.parametrize("lat,n", [("E8", 128), ("E8", 64), ("A2", 128)])
def test_kv_zero_vectors(lat, n):
    # all-zero KV vectors (padding): their step is +0 and the dithered codes
    # decode to signed zeros; full encode + decode parity
    x = workloads.gaussian(64 * 3 + 5, n, key=41)
    x[::7] = 0.0
    x[64:70] = 0.0
    check_full(x, n, lat, 2.0, seed=13, kv=True, dtype="bf16")


@pytest.mark.parametrize("tile,kv", [(256, False), (128, False), (64, False), (128, True)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tiny_and_huge_tiles(tile, kv, dtype):
    # tiles whose energy estimate is out of its range (tiny or huge rows,
    # bf16 subnormals) take the pinned sum; steps near the bottom of the
    # valid range decode through the folded scale
    x = workloads.gaussian(64 * 2 + 9, tile, key=43)
    for r, sc in enumerate((2.0 ** -40, 2.0 ** -60, 2.0 ** -64, 2.0 ** -75, 2.0 ** -100, 2.0 ** -128,
                            2.0 ** 60, 2.0 ** 100, 2.0 ** 120)):
        x[3 * r] *= np.float32(sc)
    check_full(x, tile, "E8", 2.0 if kv else 4.0, seed=17, kv=kv, dtype=dtype)


@pytest.mark.parametrize("tile,dtype", [(256, "bf16"), (128, "bf16"), (64, "f32")])
def test_every_step_significand(tile, dtype):
    # rows scaled by 2^(i / 256) over three octaves, and by large and small
    # powers of two: the tiles' steps take all 128 bf16 significands, each
    # through the encoder's reciprocal of the step
    T = 3 * 256 + 64
    x = workloads.gaussian(T, tile, key=47)
    x /= np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=1, keepdims=True)).astype(np.float32)
    sc = np.exp2(np.arange(T, dtype=np.float64) / 256.0 - 1.0)
    sc[768:] *= np.exp2(np.repeat([-100.0, -40.0, 30.0, 55.0], 16))
    x *= sc[:, None].astype(np.float32)
    _, e = check_full(x, tile, "E8", 4.0, seed=19, kv=False, dtype=dtype)
    assert len(set((e.step[e.step != 0] & 0x7F).tolist())) == 128


def test_repeatable_and_workspace_reuse():
    # the ticket counter and look-back tags reset themselves between calls of
    # different sizes sharing one workspace
    # (tile and rate change the chunks staged per ticket, hence the ticket count)
    for T, tile, bps in ((320, 128, 4.0), (64 * 300 + 17, 128, 4.0), (70, 128, 4.0), (64 * 40, 128, 4.0),
                         (64 * 9 + 3, 256, 8.0), (64 * 5, 256, 2.0), (64 * 13, 128, 4.0)):
        x = workloads.gaussian(T, tile, key=T)
        xd, _ = to_device(x, "bf16")
        outs = [gpu_encode(xd, tile, "E8", bps, 5, False)[1] for _ in range(3)]
        for o in outs[1:]:
            for k in ("step", "meta", "off", "payload"):
                np.testing.assert_array_equal(o[k], outs[0][k])
        check_full(x, tile, "E8", bps, seed=5, kv=False, dtype="bf16")


def test_decoder_on_oracle_streams_and_corruption():
    _dev()
    n, lat = 128, "E8"
    x = workloads.gaussian(200, n, key=21)
    c = rate_c(lat, n, 4.0)
    e = oracle.encode(x, n, lat, c, 4)
    rng = np.random.default_rng(0)
    for trial in range(16):
        pay = e.payload.copy()
        meta = e.meta.copy()
        off = e.chunk_off.copy()
        step = e.step.copy()
        if trial % 4 == 0:
            for _ in range(3):
                w = rng.integers(0, pay.size)
                pay[w] ^= np.uint32(1) << np.uint32(rng.integers(0, 32))
        elif trial % 4 == 1:
            meta[rng.integers(0, meta.size)] += np.uint16(8 * int(rng.integers(1, 4)))
        elif trial % 4 == 2:
            off[1 + rng.integers(0, off.size - 1)] -= 1
        else:                                                # a non-finite step: corrupt tile
            step[rng.integers(0, step.size)] = (0x7F80, 0xFF80, 0x7FC0, 0x7F81)[trial // 4]
        ee = oracle.Encoded(step, meta, off, pay, 0)
        ref, st = oracle.decode(ee, 200, n, n, lat, c, 4, oracle.F32)
        h = hq.HQTensor(torch.from_numpy(pay.view(np.int32)).to(_dev()),
                        torch.from_numpy(step.view(np.int16)).to(_dev()),
                        torch.from_numpy(meta.view(np.int16)).to(_dev()),
                        torch.from_numpy(off.view(np.int32)).to(_dev()),
                        torch.zeros(1, dtype=torch.int32, device=_dev()), (200, n), torch.float32, n, lat, 4.0, 4)
        out = hq.decode(h)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))
        assert (h.flags() == hq.FLAG_CORRUPT) == (st == oracle.ECORRUPT)


# ---------------------------------------------------------------- benchmark configurations
def test_config0_full():
    check_full(workloads.config_tensor(0), 128, "E8", 4.0, seed=0, kv=False, dtype="f32")


def test_config1_full():
    check_full(workloads.config_tensor(1), 128, "E8", 4.0, seed=1, kv=False, dtype="bf16")


# The MLP weight sweep, the KV cache, the DiT stack (both drawings) and the
# tensor past 2^31 scalars are compared chunk by chunk in test_gpu_full_parity.
