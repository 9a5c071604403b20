"""Pins of the oracle's KV rotation by a Haar-uniform orthogonal matrix
(gist.science explainer of HyperQuant, Methodology section 4, "Bias
Correction for KV Cache": a per-layer Haar rotation as the alternative to the
sign diagonal).  Each output is one ascending fused multiply-add chain."""
import numpy as np
import torch

import oracle
from kv_cache_tile_amd import workloads

D = 128


def _x(rows, key=11):
    return np.random.default_rng(key).standard_normal((rows, D)).astype(np.float32)


def test_identity_and_signed_permutation_are_exact():
    x = _x(5)
    assert np.array_equal(oracle.rotate(np.eye(D, dtype=np.float32), x), x)
    rng = np.random.default_rng(3)
    perm = rng.permutation(D)
    sg = rng.choice([-1.0, 1.0], D).astype(np.float32)
    P = np.zeros((D, D), np.float32)
    P[np.arange(D), perm] = sg                       # (P x)_i = s_i x_perm(i): not symmetric
    np.testing.assert_array_equal(oracle.rotate(P, x), x[:, perm] * sg)
    np.testing.assert_array_equal(oracle.rotate(P, x, transpose=True), (x @ P.astype(np.float64)).astype(np.float32))


def test_transpose_flag_reads_the_transpose():
    Q = workloads.haar_orthogonal(D, 1)
    x = _x(4)
    np.testing.assert_array_equal(oracle.rotate(Q, x, transpose=True), oracle.rotate(np.ascontiguousarray(Q.T), x))


def test_fma_chain_error_bound_and_orthogonality():
    Q = workloads.haar_orthogonal(D, 2)
    q64 = Q.astype(np.float64)
    assert np.abs(q64 @ q64.T - np.eye(D)).max() < 1e-6
    x = _x(64)
    y = oracle.rotate(Q, x).astype(np.float64)
    ref = x.astype(np.float64) @ q64.T
    bound = D * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(q64).T)   # gamma_d * sum |terms|
    assert np.all(np.abs(y - ref) <= bound)
    back = oracle.rotate(Q, oracle.rotate(Q, x), transpose=True).astype(np.float64)
    assert np.abs(back - x).max() < 1e-4


def test_ascending_order_is_pinned():
    # 1 + 1e8 rounds back to 1e8 (ulp 8) and then cancels: ascending gives
    # exactly 0, the descending order would give 1
    M = np.zeros((D, D), np.float32)
    M[0, :3] = 1.0
    x = np.zeros((1, D), np.float32)
    x[0, :3] = [1.0, 1e8, -1e8]
    assert oracle.rotate(M, x)[0, 0] == 0.0
    x[0, :3] = [-1e8, 1e8, 1.0]
    assert oracle.rotate(M, x)[0, 0] == 1.0


def test_bf16_in_and_out():
    Q = workloads.haar_orthogonal(D, 3)
    xb = workloads.bf16_bits(torch.from_numpy(_x(8)).to(torch.bfloat16))
    xf = (xb.astype(np.uint32) << 16).view(np.float32)
    y32 = oracle.rotate(Q, xb)
    np.testing.assert_array_equal(y32, oracle.rotate(Q, xf))
    yb = oracle.rotate(Q, xb, out_dtype=oracle.BF16)
    np.testing.assert_array_equal(yb, workloads.bf16_bits(torch.from_numpy(y32).to(torch.bfloat16)))
