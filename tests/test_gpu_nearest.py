"""The lattice quantiser alone (hq_nearest) against the oracle, bit for bit:
random blocks over several scales, half-integer and near-half inputs, the
dither domain, and (E8) two million blocks of which half lie near the
bisector of a D8 point and a neighbouring D8 + 1/2 point, where the kernel
leaves its fast decision for the two squared distances themselves."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_tile_amd import workloads

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from kv_cache_tile_amd import hq
    hq.lib()

DIM = {"Z": 1, "A2": 2, "D4": 4, "E8": 8}


def _dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def blocks(d, n, key):
    rng = np.random.default_rng(key)
    t = rng.standard_normal((n, d)) * 10.0 ** rng.uniform(-2, np.log10(250.0), (n, 1))
    k = n // 4
    t[:k] = np.round(t[:k] * 2) / 2                                    # integers and halves
    t[k:2 * k] = np.round(t[k:2 * k]) + rng.choice([-0.5, 0.5, 0.0], (k, d)) \
        + rng.choice([0.0, 2.0 ** -20, -2.0 ** -20], (k, d))           # next to halves
    t[2 * k:3 * k] = np.floor(rng.random((k, d)) * 2.0 ** 24) * 2.0 ** -23 - 1.0   # the dither box
    return t.astype(np.float32)


@pytest.mark.parametrize("lat", ["Z", "A2", "D4", "E8"])
def test_nearest_matches_oracle(lat):
    dev = _dev()
    d = DIM[lat]
    t = blocks(d, 1 << 18, key=d)
    if lat == "E8":
        t = np.concatenate([t, np.concatenate([blocks(8, 1 << 20, key=80), workloads.e8_near_ties(1 << 20, key=2)])])
    print(f"[case] nearest {lat} blocks={len(t)}", flush=True)
    got = hq.nearest(lat, torch.from_numpy(t).to(dev)).cpu().numpy()
    _, _, ref = oracle.nearest_batch(lat, t)
    # as values: a zero coordinate's sign is not part of the point (the codes
    # are integers), and the two sides form it differently
    np.testing.assert_array_equal(got, ref)


def test_nearest_argument_checks():
    dev = _dev()
    t = torch.zeros(16, 8, device=dev)
    for bad in (0, 3, 16):
        assert hq.lib().hq_nearest(bad, t.data_ptr(), 2, t.data_ptr(), None) == -1
    assert hq.lib().hq_nearest(8, None, 2, t.data_ptr(), None) == -1
    assert hq.lib().hq_nearest(8, t.data_ptr(), 0, t.data_ptr(), None) == 0
