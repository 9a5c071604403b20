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
"""
import numpy as np
import scipy.linalg

import oracle

DIM = {"Z": 1, "A2": 2, "D4": 4, "E8": 8}


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
    D = np.where(oracle.sign_bits(seed, n) == 1, -1.0, 1.0)
    d = DIM[lattice]
    out = []
    for t, (cos, syms, _) in enumerate(tiles):
        P = points(lattice, cos, syms)
        if dither:
            P = P - np.concatenate([oracle.dither_block(lattice, seed, t * n + b).astype(np.float64)
                                    for b in range(0, n, d)])
        s = np.array([int(step[t]) << 16], np.uint32).view(np.float32)[0]
        out.append(D * (H @ (P * float(s))) / np.sqrt(n))
    return np.concatenate(out)
