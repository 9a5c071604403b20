"""Where the entropy-coded, unbounded lattice codec gains over a fixed-rate,
finite codebook at the same rate (oracle-only analysis script).

The pages credit the codec's advantage over fixed-rate schemes with two
parts (gist.science explainer of HyperQuant, Key Contributions, "Superior
Weight Quantization", and Problem Statement): bits that fixed-length indices
waste (entropy slack, said to dominate at low rates), and the benefit of an
unbounded codebook over a finite one (said to dominate at high rates).  This
script measures both on seeded N(0, 1) data, which is what the per-tile RHT
makes each coordinate look like (Methodology section 1):

  - ours: the oracle's codec (Z and E8 lattices, frozen rate constants):
    payload bits per scalar, the empirical entropy of its Rice symbols, and
    the NMSE of its reconstruction;
  - fixed: a fixed-rate finite codebook of our own, the uniform quantizer
    with 2^R levels (k + 1/2) s, k = -2^(R-1) .. 2^(R-1) - 1, whose step s is
    searched for the least MSE; its indices cost exactly R bits, their
    entropy H_fixed is lower.

Decomposition at rate R, in bits (distortion ratios converted at 6.02 dB per
bit, the high-rate slope):
  gain      = (1/2) log2(D_fixed / D_ours)
  slack     = R - H_fixed                (what entropy coding the same
                                           fixed-rate indices would save)
  unbounded = gain - slack              (the rest: unbounded codebook,
                                           entropy-coded step choice, lattice)

A second fixed-rate scheme is the codec itself, clamped (fixed_rate_codec):
the same RHT, per-tile step and nearest lattice point, but the integer code
clamped to a finite codebook and stored at a fixed length, R bits per scalar:
  - Z: the code clipped to [-2^(R-1), 2^(R-1) - 1], R bits;
  - E8 (a block's code is the coset bit p and d in D8, point d + p/2): p raw,
    d0..d6 clipped to R-bit two's complement, and d7's half (d7 >> 1, its
    parity being that of d0 + ... + d6) clipped to R - 1 bits:
    1 + 7R + (R - 1) = 8R bits a block.
Its rate constant is searched for the least NMSE; its slack and the rest of
the gain are reported beside the uniform codebook's.

Only ``oracle/`` is called.  Run:  python oracle/decomposition.py
"""
from __future__ import annotations

import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import oracle  # noqa: E402

RATE_TABLE = os.path.join(os.path.dirname(HERE), "kv_cache_tile_amd", "rate_table.json")


def table_c(lat: str, tile: int, R: float) -> float:
    for e in json.load(open(RATE_TABLE))["entries"]:
        if e["lattice"] == lat and e["tile"] == tile and e["dither"] == 0 and e["bps"] == R:
            return float(np.array([int(e["c_bits"], 16)], np.uint32).view(np.float32)[0])
    raise KeyError((lat, tile, R))


def entropy_bits(codes: np.ndarray) -> float:
    """Empirical entropy (bits per symbol) of an integer array."""
    _, counts = np.unique(codes, return_counts=True)
    p = counts / counts.sum()
    return float(-(p * np.log2(p)).sum())


def symbol_entropy(lat: str, sym: np.ndarray) -> float:
    """Bits per scalar an ideal entropy coder of a lattice code's symbols
    (one row a block) would spend: Z one source; E8 the first seven
    coordinates as one source, the halved last one as another, plus the raw
    coset bit of each block."""
    if lat == "Z":
        return entropy_bits(sym.ravel())
    return (7 * entropy_bits(sym[:, :7].ravel()) + entropy_bits(sym[:, 7]) + 1.0) / 8.0


def fixed_rate_uniform(x: np.ndarray, R: int, grid: int = 400):
    """The 2^R-level uniform quantizer with the least MSE on x (step searched
    on a fine grid, then refined): (step, MSE, index entropy)."""
    L = 1 << R
    x = x.astype(np.float64).ravel()

    def mse_of(s):
        k = np.clip(np.floor(x / s), -L // 2, L // 2 - 1)
        return float(np.mean((x - (k + 0.5) * s) ** 2)), k

    lo, hi = 0.2 * 8.0 / L, 3.0 * 8.0 / L
    for _ in range(3):
        steps = np.linspace(lo, hi, grid // 4)
        errs = [mse_of(s)[0] for s in steps]
        i = int(np.argmin(errs))
        lo, hi = steps[max(i - 1, 0)], steps[min(i + 1, len(steps) - 1)]
    s = 0.5 * (lo + hi)
    m, k = mse_of(s)
    return s, m, entropy_bits(k.astype(np.int64))


def ours(x: np.ndarray, lat: str, tile: int, R: float, seed: int = 5):
    """The oracle codec on x [rows][tile]: (payload bps, symbol entropy per
    scalar, NMSE).  Symbol entropy: the Rice symbols of every tile (zigzag of
    the lattice's integer coordinates, E8's last one halved first, the
    parity strip) as i.i.d. sources (symbol_entropy), plus E8's raw coset
    bit per 8 scalars: what an ideal entropy coder of the same symbols would
    spend."""
    c = table_c(lat, tile, R)
    e = oracle.encode(x, tile, lat, c, seed)
    bps = float((e.meta >> 3).astype(np.int64).sum()) / x.size
    xh, st = oracle.decode(e, x.shape[0], x.shape[1], tile, lat, c, seed, oracle.F32)
    nmse = float(((xh.astype(np.float64) - x) ** 2).sum() / (x.astype(np.float64) ** 2).sum())
    codes, cos = [], []
    for r in range(x.shape[0]):
        y = oracle.rht_forward(x[r], seed)
        s, _ = oracle.tile_step(y, c)
        inv = np.float32(0.0) if s == 0 else np.float32(1.0) / s
        t = (y * inv).astype(np.float32)
        p, d, _ = oracle.nearest_batch(lat, t)
        if lat == "E8":
            d = d.copy()
            d[:, 7] >>= 1                      # the stripped parity bit
        sym = np.where(d >= 0, 2 * d, -2 * d - 1)   # zigzag
        codes.append(sym.reshape(-1, 8 if lat == "E8" else 1))
        cos.append(p)
    h = symbol_entropy(lat, np.concatenate(codes))
    return bps, h, nmse


def clamp_codes(lat: str, p: np.ndarray, d: np.ndarray, R: int):
    """The fixed-rate codebook of the clamped codec: (points, symbols) of the
    clamped codes (see the module text); symbols as coded, one row a block."""
    lo, hi = -(1 << (R - 1)), (1 << (R - 1)) - 1
    if lat == "Z":
        dc = np.clip(d, lo, hi)
        return dc.astype(np.float64), dc
    dc = d.astype(np.int64).copy()
    dc[:, :7] = np.clip(dc[:, :7], lo, hi)
    h7 = np.clip(d[:, 7].astype(np.int64) >> 1, -(1 << (R - 2)), (1 << (R - 2)) - 1)
    dc[:, 7] = 2 * h7 + (dc[:, :7].sum(axis=1) & 1)
    sym = np.concatenate([dc[:, :7], h7[:, None]], axis=1)
    return dc + p[:, None] / 2.0, sym


def fixed_rate_codec(x: np.ndarray, lat: str, tile: int, R: int, seed: int = 5, grid: int = 24):
    """The codec clamped to a fixed-rate codebook (module text) on x
    [rows][tile], at the rate constant of least NMSE: (c, NMSE, entropy of
    its symbols per scalar, bits per scalar).  The error is measured in the
    rotated domain (the RHT is orthogonal)."""
    ys = np.stack([oracle.rht_forward(r, seed) for r in x]).astype(np.float32)
    d_ = 8 if lat == "E8" else 1
    energy = float((ys.astype(np.float64) ** 2).sum())

    def run(c):
        pts, syms = [], []
        for y in ys:
            s, _ = oracle.tile_step(y, c)
            inv = np.float32(0.0) if s == 0 else np.float32(1.0) / s
            p, d, _ = oracle.nearest_batch(lat, (y * inv).astype(np.float32))
            P, sym = clamp_codes(lat, p, d.reshape(-1, d_), R)
            pts.append(P.reshape(-1) * float(s))
            syms.append(sym.reshape(-1))
        err = float(((np.stack(pts) - ys.astype(np.float64)) ** 2).sum())
        return err / energy, np.concatenate(syms)

    c_hr = float(np.array([oracle.RATE_K_BITS[lat]], np.uint32).view(np.float32)[0]) * 2.0 ** -R
    lo, hi = 0.5 * c_hr, 3.0 * c_hr
    for _ in range(3):
        cs = np.geomspace(lo, hi, grid)
        errs = [run(float(np.float32(c)))[0] for c in cs]
        i = int(np.argmin(errs))
        lo, hi = cs[max(i - 1, 0)], cs[min(i + 1, grid - 1)]
    c = float(np.float32(np.sqrt(lo * hi)))
    nmse, syms = run(c)
    h = symbol_entropy(lat, syms.reshape(-1, d_))
    bits = float(R) if lat == "Z" else (1 + 7 * R + (R - 1)) / 8.0
    return c, nmse, h, bits


def decomposition(R: int, n_rows: int = 512, tile: int = 256, key: int = 11):
    x = np.random.Generator(np.random.PCG64(np.random.SeedSequence([key, R]))).standard_normal(
        (n_rows, tile)).astype(np.float32)
    s, d_fixed, h_fixed = fixed_rate_uniform(x, R)
    out = {"R": R, "fixed_step": s, "fixed_nmse": d_fixed / float(np.mean(x.astype(np.float64) ** 2)),
           "fixed_entropy": h_fixed}
    for lat in ("Z", "E8"):
        bps, h, nmse = ours(x, lat, tile, float(R))
        out[lat] = {"bps": bps, "entropy": h, "nmse": nmse,
                    "gain_bits": 0.5 * math.log2(out["fixed_nmse"] / nmse)}
    out["slack_bits"] = R - h_fixed
    for lat in ("Z", "E8"):
        out[lat]["unbounded_bits"] = out[lat]["gain_bits"] - out["slack_bits"]
        # the codec clamped to a fixed-rate codebook of the same lattice
        c, nmse_f, h_f, bits = fixed_rate_codec(x, lat, tile, R)
        gain = 0.5 * math.log2(nmse_f / out[lat]["nmse"])
        out[lat]["clamped"] = {"c": c, "bits": bits, "nmse": nmse_f, "entropy": h_f, "slack_bits": bits - h_f,
                               "gain_bits": gain, "unbounded_bits": gain - (bits - h_f)}
    return out


def main_clamped():
    print("| R | lattice | clamped codec: NMSE, index entropy | slack | ours: Rice bps, NMSE | gain = slack + rest |")
    print("|---|---|---|---|---|---|")
    for R in (2, 3, 4, 5, 6):
        o = decomposition(R)
        for lat in ("Z", "E8"):
            f, u = o[lat]["clamped"], o[lat]
            print(f"| {R} | {lat} | {f['nmse']:.4e}, {f['entropy']:.3f} | {f['slack_bits']:.3f} | "
                  f"{u['bps']:.3f}, {u['nmse']:.4e} | {f['gain_bits']:.3f} = {f['slack_bits']:.3f} + "
                  f"{f['unbounded_bits']:.3f} |", flush=True)


def main():
    print("| R | fixed-rate NMSE | its index entropy | slack (bits) | Z: Rice bps, symbol entropy, NMSE | Z gain = slack + rest | E8: Rice bps, symbol entropy, NMSE | E8 gain = slack + rest |")
    print("|---|---|---|---|---|---|---|---|")
    for R in (2, 3, 4, 5, 6):
        o = decomposition(R)
        z, e = o["Z"], o["E8"]
        print(f"| {R} | {o['fixed_nmse']:.4e} | {o['fixed_entropy']:.3f} | {o['slack_bits']:.3f} | "
              f"{z['bps']:.3f}, {z['entropy']:.3f}, {z['nmse']:.4e} | {z['gain_bits']:.3f} ({o['slack_bits']:.3f} + {z['unbounded_bits']:.3f}) | "
              f"{e['bps']:.3f}, {e['entropy']:.3f}, {e['nmse']:.4e} | {e['gain_bits']:.3f} ({o['slack_bits']:.3f} + {e['unbounded_bits']:.3f}) |",
              flush=True)


if __name__ == "__main__":
    main_clamped() if "--clamped" in sys.argv else main()
