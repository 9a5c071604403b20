"""Pins of the oracle's nearest-lattice-point decoders (gist.science explainer of
HyperQuant, Methodology section 2): brute force over a neighbourhood,
lattice membership, translation invariance, covering radius, the textbook
normalized second moments, and the E8 root system."""
import itertools

import numpy as np
import pytest

import oracle
from hq_testutil import golden_json
from kv_cache_tile_amd import workloads

CONST = golden_json("lattice_constants.json")
DIM = {"Z": 1, "A2": 2, "D4": 4, "E8": 8}
S3 = np.sqrt(3.0)


def candidates(lat, t, r):
    """All lattice points whose coordinates lie within about r of t (fp64)."""
    d = DIM[lat]
    if lat == "A2":
        pts = []
        for p in (0, 1):
            m0 = np.floor(t[0] - p / 2)
            n0 = np.floor(t[1] / S3 - p / 2)
            for dm in range(-r - 1, r + 2):
                for dn in range(-r - 1, r + 2):
                    pts.append(((m0 + dm + p / 2), S3 * (n0 + dn + p / 2)))
        return np.array(pts)
    offs = np.array(list(itertools.product(range(-r, r + 1), repeat=d)), np.float64)
    out = []
    for p in ((0, 1) if lat == "E8" else (0,)):
        base = np.round(t - p / 2.0)
        z = base + offs
        if lat in ("D4", "E8"):
            z = z[(z.sum(axis=1) % 2) == 0]
        out.append(z + p / 2.0)
    return np.concatenate(out)


def member(lat, code_p, ints):
    if lat == "Z" or lat == "A2":
        return True
    if lat == "D4":
        return int(ints.sum()) % 2 == 0
    return code_p in (0, 1) and int(ints.sum()) % 2 == 0


def rand_inputs(d, n, seed):
    rng = np.random.default_rng(seed)
    scale = 10.0 ** rng.uniform(-1, 2, size=(n, 1))
    t = rng.standard_normal((n, d)) * scale
    # crafted ties and near-ties: half-integers, integers, small perturbations
    k = n // 4
    t[:k] = np.round(t[:k] * 2) / 2
    t[k:2 * k] = np.round(t[k:2 * k]) + rng.choice([-0.5, 0.5, 0.0], size=(k, d)) \
        + rng.choice([0, 1e-6, -1e-6], size=(k, d))
    return t.astype(np.float32)


TOL = {"Z": 1e-9, "D4": 1e-9, "E8": 1e-5, "A2": 2e-4}


@pytest.mark.parametrize("lat", ["Z", "A2", "D4", "E8"])
def test_nearest_point_matches_brute_force(lat):
    d = DIM[lat]
    t = rand_inputs(d, 400, seed=d)
    ps, ints, pts = oracle.nearest_batch(lat, t)
    for i in range(len(t)):
        tt = t[i].astype(np.float64)
        cand = candidates(lat, tt, 1)
        best = np.min(((cand - tt) ** 2).sum(axis=1))
        # the oracle's point, recomputed in fp64 from its integer code
        if lat == "A2":
            P = np.array([ints[i, 0] + ps[i] / 2, S3 * (ints[i, 1] + ps[i] / 2)])
        else:
            P = ints[i].astype(np.float64) + ps[i] / 2.0
        np.testing.assert_allclose(pts[i], P, rtol=1e-6, atol=1e-6)
        dist = ((P - tt) ** 2).sum()
        assert member(lat, ps[i], ints[i])
        assert dist <= best + TOL[lat] * max(1.0, np.abs(tt).max()), (lat, tt, P, dist, best)


@pytest.mark.parametrize("lat", ["D4", "E8"])
def test_nearest_point_wide_neighbourhood(lat):
    # radius-2 box: does not rely on the covering radius to bound the search
    t = rand_inputs(DIM[lat], 12, seed=99)
    ps, ints, _ = oracle.nearest_batch(lat, t)
    for i in range(len(t)):
        tt = t[i].astype(np.float64)
        cand = candidates(lat, tt, 2)
        best = np.min(((cand - tt) ** 2).sum(axis=1))
        P = ints[i] + ps[i] / 2.0
        assert ((P - tt) ** 2).sum() <= best + TOL[lat]


def test_z_is_numpy_rint():
    t = rand_inputs(1, 2000, seed=5)
    _, ints, pts = oracle.nearest_batch("Z", t)
    np.testing.assert_array_equal(pts[:, 0], np.rint(t[:, 0]))


@pytest.mark.parametrize("lat", ["A2", "D4", "E8"])
def test_translation_invariance_and_covering_radius(lat):
    d = DIM[lat]
    rng = np.random.default_rng(3)
    t = (rng.standard_normal((300, d)) * 3).astype(np.float32)
    if lat == "E8":
        lams = [np.eye(8)[0] * 2, np.full(8, 0.5), np.eye(8)[0] + np.eye(8)[1]]
    elif lat == "D4":
        lams = [np.eye(4)[0] * 2, np.eye(4)[0] + np.eye(4)[3]]
    else:
        lams = [np.array([1.0, 0.0]), np.array([0.5, S3 / 2])]
    _, _, p0 = oracle.nearest_batch(lat, t)
    r = CONST["covering_radius"][lat]
    assert np.all(np.sqrt(((p0 - t) ** 2).sum(axis=1)) <= r + 1e-5)
    for lam in lams:
        _, _, p1 = oracle.nearest_batch(lat, (t + lam).astype(np.float32))
        # skip the few inputs whose fp32 shift is inexact or near a tie
        ok = np.abs(((t + lam).astype(np.float32) - t) - lam).max(axis=1) < 1e-6
        np.testing.assert_allclose(p1[ok], (p0 + lam)[ok], atol=1e-4)


@pytest.mark.parametrize("lat", ["Z", "A2", "D4", "E8"])
def test_normalized_second_moment(lat):
    # t uniform on a fundamental region of a sublattice => the error is uniform
    # on the Voronoi cell; G = E|e|^2 / (d V^(2/d))  (Conway & Sloane)
    d = DIM[lat]
    rng = np.random.default_rng(2026)
    N = 1 << 20
    if lat == "A2":
        t = np.stack([rng.random(N), S3 * rng.random(N)], axis=1)
    elif lat == "Z":
        t = rng.random((N, 1))
    else:
        t = 2.0 * rng.random((N, d))
    t = t.astype(np.float32)
    _, _, p = oracle.nearest_batch(lat, t)
    e2 = ((p.astype(np.float64) - t) ** 2).sum(axis=1).mean()
    V = CONST["covolume"][lat]
    G = e2 / (d * V ** (2.0 / d))
    assert abs(G - CONST["normalized_second_moment"][lat]) < 5e-4, G
    # and the ordering the pages rely on: every lattice beats scalar rounding
    assert G <= CONST["normalized_second_moment"]["Z"] + 5e-4


def e8_roots():
    roots = []
    for i, j in itertools.combinations(range(8), 2):
        for si in (-1, 1):
            for sj in (-1, 1):
                v = np.zeros(8); v[i] = si; v[j] = sj
                roots.append(v)
    for signs in itertools.product((-0.5, 0.5), repeat=8):
        if sum(1 for s in signs if s < 0) % 2 == 0:
            roots.append(np.array(signs))
    return np.array(roots)


def test_e8_roots_are_fixed_points():
    R = e8_roots()
    assert len(R) == CONST["kissing_number"]["E8"]
    assert np.allclose((R ** 2).sum(axis=1), CONST["minimal_norm_squared"]["E8"])
    ps, ints, pts = oracle.nearest_batch("E8", R.astype(np.float32))
    np.testing.assert_array_equal(pts, R.astype(np.float32))
    # small perturbations stay with the root (packing radius sqrt2/2)
    rng = np.random.default_rng(1)
    Rp = R + rng.uniform(-0.2, 0.2, R.shape) / np.sqrt(8)
    _, _, pts2 = oracle.nearest_batch("E8", Rp.astype(np.float32))
    np.testing.assert_array_equal(pts2, R.astype(np.float32))


def test_d4_minimal_vectors():
    v = []
    for i, j in itertools.combinations(range(4), 2):
        for si in (-1, 1):
            for sj in (-1, 1):
                x = np.zeros(4); x[i] = si; x[j] = sj
                v.append(x)
    v = np.array(v)
    assert len(v) == CONST["kissing_number"]["D4"]
    _, _, p = oracle.nearest_batch("D4", v.astype(np.float32))
    np.testing.assert_array_equal(p, v)


@pytest.mark.parametrize("lat", ["Z", "A2", "D4", "E8"])
def test_dither_is_uniform_on_the_voronoi_cell(lat):
    # Methodology section 4: U ~ Uniform(V(Lambda)).  Second moment of the
    # cell = G V^(2/d) per dimension; mean zero; U is its own nearest-point error.
    d = DIM[lat]
    N = 20000
    u = np.array([oracle.dither_block(lat, 5, g * d) for g in range(N)], np.float64)
    V = CONST["covolume"][lat]
    want = CONST["normalized_second_moment"][lat] * V ** (2.0 / d)
    assert abs((u ** 2).sum(axis=1).mean() / d - want) < 4 * want / np.sqrt(N) * 2
    assert np.all(np.abs(u.mean(axis=0)) < 0.02)
    _, _, p = oracle.nearest_batch(lat, u.astype(np.float32))
    assert np.mean(np.abs(p).max(axis=1) == 0) > 0.999     # Q(U) = 0 up to boundary ties


def e8_coset_points(t32):
    """Both candidates of Conway & Sloane's E8 decoder, written here in numpy
    (fp64 on the fp32 inputs): A the nearest point of D8, B of D8 + 1/2
    (round; with an odd sum of integer parts move the coordinate farthest from
    the rounded point, the first on ties, one step towards t).  Distances to
    the rounded point are exact here through |t - rint t|: for B the farthest
    coordinate is the one nearest an integer."""
    t = t32.astype(np.float64)
    rows = np.arange(len(t))
    ad = np.abs(t - np.rint(t))
    out = []
    for half in (False, True):
        base = np.floor(t) if half else np.rint(t)
        P = base + (0.5 if half else 0.0)
        odd = (base.sum(axis=1).astype(np.int64) % 2) == 1
        j = np.argmin(ad, axis=1) if half else np.argmax(ad, axis=1)   # the first of them
        step = np.where(t[rows, j] >= P[rows, j], 1.0, -1.0)
        P[rows[odd], j[odd]] += step[odd]
        out.append(P)
    return out


def test_e8_choice_is_the_nearer_coset_point():
    # The oracle's E8 point is the nearer of the two coset candidates: on 2^20
    # random blocks (|t| up to about 250, the largest the codec quantises) and
    # 2^20 blocks near a tie between neighbouring points of the two cosets, it
    # is one of the two candidates (written independently here), and its exact
    # (fp64) squared distance is at most the other's plus the error bound of
    # the fp32 evaluation of the distance difference (10 * 2^-23); away from
    # that band the choice is the exact one, and ties on an exact grid go to D8.
    rng = np.random.default_rng(8)
    N = 1 << 20
    t = (rng.standard_normal((N, 8)) * 10.0 ** rng.uniform(-1, np.log10(250.0), (N, 1))).astype(np.float32)
    ties = workloads.e8_near_ties(N, key=1)
    T = np.concatenate([t, ties])
    p, ints, pts = oracle.nearest_batch("E8", T)
    A, B = e8_coset_points(T)
    isA = np.all(pts == A, axis=1)
    isB = np.all(pts == B, axis=1)
    assert np.all(isA | isB)
    np.testing.assert_array_equal(p == 1, isB & ~isA)
    t64 = T.astype(np.float64)
    dA = ((t64 - A) ** 2).sum(axis=1)
    dB = ((t64 - B) ** 2).sum(axis=1)
    bound = 10 * 2.0 ** -23
    chosen = np.where(p == 1, dB, dA)
    other = np.where(p == 1, dA, dB)
    assert np.all(chosen <= other + bound)
    far = np.abs(dA - dB) > bound
    np.testing.assert_array_equal((p == 1)[far], (dB < dA)[far])
    assert far[:N].mean() > 0.999 and (~far[N:]).sum() > N // 8     # the crafted blocks reach the band
    grid_ties = (np.arange(2 * N) >= N) & (np.arange(2 * N) < N + N // 4)   # exact ties on a 1/4 grid
    assert np.all(dA[grid_ties] == dB[grid_ties]) and np.all(p[grid_ties] == 0)
