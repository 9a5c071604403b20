"""Independent reader of the compressed stream, written from the format's
description alone (a second implementation that pins the oracle's layout).

Format: per tile t (row-major tile order) a bf16 step s_t and a 16-bit meta
word (len << 3 | k); tiles are grouped 64 to a chunk, chunk c starts at 32-bit
word chunk_off[c] of the payload; inside a chunk tiles are bit-contiguous
(bit b = bit b%32 of word b//32).  A tile is its coset bits (E8: one per
8-block, A2: one per 2-block), then the n k-bit remainders (least significant
bit first), then the n unary quotients (q zero bits, then a one bit); the
symbol is (q<<k)|r.
Symbols are zigzag codes (v >= 0 -> 2v, v < 0 -> -2v-1).  E8 and D4 store the
last coordinate of a block halved (floor), its parity being that of the sum
of the others.  Reconstruction (fp64 here): point = code (+1/2 for coset 1;
A2: (m + p/2, sqrt3 (n' + p/2))), minus the dither for the KV variant, times
s, then x = D H v / sqrt(n).

The sign diagonal and the dither are regenerated here too, from their
description, with no call into the oracle: a counter-based generator, the
"pcg" hash of Jarzynski & Olano (JCGT 2020: one step of the PCG32 linear
congruential generator, multiplier 747796405 and increment 2891336453, then
PCG's RXS-M-XS output permutation with multiplier 277803737); per call two
keys hash(hash(lo32(seed) ^ domain) ^ hi32(seed)) for the domains "SIGN"
and "DITH" (their ASCII codes as big-endian words); D_ii = -1 iff the top
bit of hash(key_sign + i) is set; coordinate g of the call (row-major)
draws a = hash(key_dith + g) >> 8, a point of the box (E8, D4: a 2^-23 - 1;
Z: a 2^-24 - 1/2; A2: (a0 2^-24 - 1/2, sqrt3 (a1 2^-24 - 1/2))), reduced
into the Voronoi cell, u = v - Q(v), with the nearest point Q written out
below (fp64).
"""
import numpy as np
import scipy.linalg

DIM = {"Z": 1, "A2": 2, "D4": 4, "E8": 8}
SIGN, DITH = 0x5349474E, 0x44495448


def pcg_hash(v):
    """The pcg hash on uint32 numpy values (wrapping arithmetic)."""
    v = np.asarray(v, dtype=np.uint32)
    with np.errstate(over="ignore"):
        state = v * np.uint32(747796405) + np.uint32(2891336453)
        word = ((state >> ((state >> np.uint32(28)) + np.uint32(4))) ^ state) * np.uint32(277803737)
    return (word >> np.uint32(22)) ^ word


def key(seed, domain):
    lo, hi = np.uint32(seed & 0xFFFFFFFF), np.uint32(seed >> 32)
    return pcg_hash(pcg_hash(lo ^ np.uint32(domain)) ^ hi)


def signs(seed, n):
    """+-1.0 entries of the sign diagonal for one tile of n."""
    with np.errstate(over="ignore"):
        h = pcg_hash(key(seed, SIGN) + np.arange(n, dtype=np.uint32))
    return np.where(h >> np.uint32(31), -1.0, 1.0)


def nearest(lattice, t):
    """Nearest lattice points of the rows of t (fp64): Z rint; D4 and the two
    cosets of E8 by Conway & Sloane's D_n rule; A2 the nearer of its two
    rectangular cosets; E8 the nearer of its two cosets (ties to D8)."""
    t = np.asarray(t, np.float64)
    rows = np.arange(len(t))

    def dn(t, half):
        base = np.floor(t) if half else np.rint(t)
        P = base + (0.5 if half else 0.0)
        odd = base.sum(axis=1).astype(np.int64) % 2 == 1
        j = np.argmax(np.abs(t - P), axis=1)
        step = np.where(t[rows, j] >= P[rows, j], 1.0, -1.0)
        P[rows[odd], j[odd]] += step[odd]
        return P

    if lattice == "Z":
        return np.rint(t)
    if lattice == "D4":
        return dn(t, False)
    if lattice == "E8":
        A, B = dn(t, False), dn(t, True)
        useB = ((t - B) ** 2).sum(axis=1) < ((t - A) ** 2).sum(axis=1)
        return np.where(useB[:, None], B, A)
    s3 = np.sqrt(3.0)
    y = t[:, 1] / s3
    A = np.stack([np.rint(t[:, 0]), s3 * np.rint(y)], axis=1)
    B = np.stack([np.floor(t[:, 0]) + 0.5, s3 * (np.floor(y) + 0.5)], axis=1)
    useB = ((t - B) ** 2).sum(axis=1) < ((t - A) ** 2).sum(axis=1)
    return np.where(useB[:, None], B, A)


def dither_values(lattice, seed, g0, n):
    """Dither of the n coordinates g0 .. g0 + n - 1 of a call, in blocks of d."""
    d = DIM[lattice]
    with np.errstate(over="ignore"):
        a = (pcg_hash(key(seed, DITH) + np.uint32(g0) + np.arange(n, dtype=np.uint32)) >> np.uint32(8))
    a = a.astype(np.float64).reshape(-1, d)
    if lattice in ("E8", "D4"):
        v = a * 2.0 ** -23 - 1.0
    else:
        v = a * 2.0 ** -24 - 0.5
        if lattice == "A2":
            v[:, 1] *= np.sqrt(3.0)
    return (v - nearest(lattice, v)).reshape(-1)


def unzz(u):
    u = np.asarray(u, np.int64)
    return np.where(u & 1, -((u + 1) >> 1), u >> 1)


def parse(step, meta, chunk_off, payload, T, n, lattice):
    d = DIM[lattice]
    nb = n // d if lattice in ("E8", "A2") else 0
    bits = np.unpackbits(np.ascontiguousarray(payload, np.uint32).view(np.uint8), bitorder="little")
    tiles = []
    C = (T + 63) // 64
    for c in range(C):
        b = int(chunk_off[c]) * 32
        for t in range(c * 64, min(T, c * 64 + 64)):
            L, k = int(meta[t]) >> 3, int(meta[t]) & 7
            b0 = b
            cos = bits[b:b + nb].astype(np.int64)
            b += nb
            syms = np.empty(n, np.int64)
            rem = bits[b:b + n * k].reshape(n, k).astype(np.int64) if k else np.zeros((n, 0), np.int64)
            r = (rem << np.arange(k)).sum(axis=1) if k else np.zeros(n, np.int64)
            b += n * k
            for i in range(n):
                q = 0
                while bits[b] == 0:
                    q += 1
                    b += 1
                b += 1
                syms[i] = (q << k) | int(r[i])
            assert b - b0 == L, "tile length differs from its meta word"
            tiles.append((cos, syms, k))
        end = int(chunk_off[c + 1]) * 32
        assert (b + 31) // 32 * 32 == end, "chunk not padded to a word"
        assert not bits[b:end].any(), "padding bits must be zero"
    return tiles


def points(lattice, cos, syms):
    d = DIM[lattice]
    blocks = syms.reshape(-1, d)
    if lattice == "Z":
        return unzz(blocks[:, 0]).astype(np.float64)
    if lattice == "A2":
        m, nn = unzz(blocks[:, 0]), unzz(blocks[:, 1])
        return np.stack([m + cos / 2.0, np.sqrt(3.0) * (nn + cos / 2.0)], axis=1).reshape(-1)
    v = unzz(blocks)
    v[:, -1] = 2 * v[:, -1] + (v[:, :-1].sum(axis=1) & 1)
    h = cos[:, None] / 2.0 if lattice == "E8" else 0.0
    return (v + h).reshape(-1).astype(np.float64)


def reconstruct(tiles, step, n, lattice, seed, dither=False):
    H = scipy.linalg.hadamard(n).astype(np.float64)
    D = signs(seed, n)
    out = []
    for t, (cos, syms, _) in enumerate(tiles):
        P = points(lattice, cos, syms)
        if dither:
            P = P - dither_values(lattice, seed, t * n, n)
        s = np.array([int(step[t]) << 16], np.uint32).view(np.float32)[0]
        out.append(D * (H @ (P * float(s))) / np.sqrt(n))
    return np.concatenate(out)
