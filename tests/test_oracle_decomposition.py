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
