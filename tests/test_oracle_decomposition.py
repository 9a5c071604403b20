"""Pins of the entropy-slack / unbounded-codebook analysis (oracle/
decomposition.py; gist.science explainer of HyperQuant, Key Contributions).
Its fixed-rate baseline must be the textbook optimum uniform quantizer of a
unit Gaussian (Max 1960, as tabulated by Jayant and Noll: step and MSE for
8, 16 and 32 levels), and its entropy estimate exact on known sources."""
import numpy as np
import pytest

import decomposition

# levels: (optimum step, its MSE) for N(0, 1)
MAX_UNIFORM = {3: (0.5860, 0.03744), 4: (0.3352, 0.01154), 5: (0.1881, 0.003490)}


@pytest.mark.parametrize("R", [3, 4, 5])
def test_fixed_rate_baseline_is_the_optimum_uniform_quantizer(R):
    x = np.random.default_rng(100 + R).standard_normal(1 << 21)
    s, mse, h = decomposition.fixed_rate_uniform(x, R)
    step, ref = MAX_UNIFORM[R]
    assert abs(s / step - 1) < 0.02 and abs(mse / ref - 1) < 0.02
    assert h < R                        # a fixed-length index leaves entropy slack


def test_entropy_estimate():
    assert decomposition.entropy_bits(np.zeros(100, np.int64)) == 0.0
    assert decomposition.entropy_bits(np.arange(1 << 10) % 16) == pytest.approx(4.0, abs=1e-12)
    p = np.array([0.5, 0.25, 0.25])
    codes = np.repeat([0, 1, 2], (p * 4000).astype(int))
    assert decomposition.entropy_bits(codes) == pytest.approx(1.5, abs=1e-12)


@pytest.mark.parametrize("R", [2, 4, 6])
def test_clamped_codebook(R):
    # the clamped E8 code stays in E8 (d in D8), in its R-bit ranges, at
    # exactly 8R bits a block; codes already in range are unchanged
    rng = np.random.default_rng(R)
    d = rng.integers(-(1 << R), 1 << R, size=(5000, 8))
    d[:, 7] += d.sum(axis=1) & 1                       # make each row a D8 point
    p = rng.integers(0, 2, 5000)
    P, sym = decomposition.clamp_codes("E8", p, d, R)
    dc = P - p[:, None] / 2.0
    assert np.all(dc.sum(axis=1) % 2 == 0)
    assert np.all(np.abs(sym[:, :7]) <= 1 << (R - 1)) and np.all(sym[:, :7] < 1 << (R - 1))
    assert np.all((sym[:, 7] >= -(1 << (R - 2))) & (sym[:, 7] < 1 << (R - 2)))
    inside = np.all((d[:, :7] >= -(1 << (R - 1))) & (d[:, :7] < 1 << (R - 1)), axis=1) & \
        ((d[:, 7] >> 1) >= -(1 << (R - 2))) & ((d[:, 7] >> 1) < 1 << (R - 2))
    np.testing.assert_array_equal(dc[inside], d[inside])
    Pz, sz = decomposition.clamp_codes("Z", np.zeros(5000, np.int64), d[:, :1], R)
    assert np.all((sz >= -(1 << (R - 1))) & (sz < 1 << (R - 1)))


def test_clamped_codec_rates_and_order():
    # the clamped codec at its best constant: R bits per scalar exactly, E8
    # below Z in distortion (granular gain; at 3 bps and below the clamped
    # E8 code's overload costs that again), and for Z near Max's optimum
    # uniform quantizer of a unit Gaussian (the RHT makes each coordinate
    # near-Gaussian; the codebook here is the 2^R integers from -2^(R-1))
    x = np.random.Generator(np.random.PCG64(np.random.SeedSequence([9, 9]))).standard_normal(
        (192, 256)).astype(np.float32)
    for R in (4, 5):
        cz, nz, hz, bz = decomposition.fixed_rate_codec(x, "Z", 256, R)
        ce, ne, he, be = decomposition.fixed_rate_codec(x, "E8", 256, R)
        assert bz == R and be == R
        assert ne < nz and hz < R and he < R
        assert abs(nz / MAX_UNIFORM[R][1] - 1) < 0.06
