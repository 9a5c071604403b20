"""Seeded synthetic inputs shaped like the workloads the pages quantize.

The pages evaluate on Llama-3.1-8B-Instruct weights and KV caches and on the
LTX-2-19B DiT (gist.science explainer of HyperQuant, "Experimental
Results"); neither the weights nor the data are available, so these seeded
tensors stand in for them, with the shapes and value distributions of the
five benchmark configurations.  This module holds random-number generation
only — none of the codec's arithmetic — so that both the HIP path and the CPU
oracle are fed from it.

All generators draw in fp64 from numpy's PCG64 (SeedSequence(key)), round to
fp32, and (for bf16 tensors) round to bf16 by round-to-nearest-even.  The
largest tensors (KV cache, DiT stack) are drawn per slice so memory stays
bounded; each slice has its own key, so any slice can be regenerated alone.
"""
from __future__ import annotations

import numpy as np
import torch


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32/fp64 numpy -> torch bfloat16 (RNE)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """torch bfloat16 tensor (any device) -> numpy uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def student_t_outlier_cols(rows: int, cols: int, key: int, nu: float = 4.0, n_out: int = 8,
                           scale: float = 20.0) -> np.ndarray:
    """Weight matrix, i.i.d. standard Student-t(nu) entries, n_out random columns
    scaled by `scale` (column set drawn before the values).  fp32."""
    rng = _rng(key)
    out_cols = rng.choice(cols, n_out, replace=False)
    w = rng.standard_t(nu, size=(rows, cols))
    w[:, out_cols] *= scale
    return w.astype(np.float32)


def gaussian_outlier_channels(rows: int, cols: int, key: int, std: float = 0.02,
                              frac: float = 0.01, scale: float = 10.0) -> np.ndarray:
    """Llama-style projection weight: N(0, std^2) entries with round(frac*cols)
    input channels (columns) scaled by `scale`.  fp32."""
    rng = _rng(key)
    k = int(round(frac * cols))
    out_cols = rng.choice(cols, k, replace=False)
    w = std * rng.standard_normal((rows, cols))
    w[:, out_cols] *= scale
    return w.astype(np.float32)


def kv_cache_entry(b: int, heads: int, seq: int, head_dim: int, key: int, which: str) -> np.ndarray:
    """Batch entry b [H, S, D] of kv_cache (each entry has a key of its own, so
    one can be drawn alone).  fp32."""
    sub = 0 if which == "K" else 1
    v = _rng(key, sub, b).standard_normal((heads, seq, head_dim))
    if which == "K":
        v *= _rng(key, 0, 99).lognormal(0.0, 1.0, size=(heads, head_dim))[:, None, :]
    return v.astype(np.float32)


def kv_cache(batch: int, heads: int, seq: int, head_dim: int, key: int, which: str) -> np.ndarray:
    """KV cache [B, H, S, D]: V ~ N(0,1); K ~ N(0,1) * scale[h, d] with a
    per-channel outlier scale ~ LogNormal(0, 1).  Drawn per batch entry.  fp32."""
    out = np.empty((batch, heads, seq, head_dim), np.float32)
    for b in range(batch):
        out[b] = kv_cache_entry(b, heads, seq, head_dim, key, which)
    return out


def dit_layer(rows: int, cols: int, key: int, layer: int, std: float = 0.02,
              p_out: float = 0.005, nu: float = 3.0) -> np.ndarray:
    """One DiT linear weight: N(0, std^2) entries, each replaced with
    probability p_out by a standard (unit-scale) Student-t(nu) draw.  fp32."""
    rng = _rng(key, layer)
    w = std * rng.standard_normal((rows, cols))
    mask = rng.random((rows, cols)) < p_out
    w[mask] = rng.standard_t(nu, size=int(mask.sum()))
    return w.astype(np.float32)


def gaussian(rows: int, cols: int, key: int) -> np.ndarray:
    return _rng(key).standard_normal((rows, cols)).astype(np.float32)


# The five benchmark configurations (0-indexed; configuration i uses key/seed i).
CONFIGS = {
    0: dict(name="weight-1024x1024-f32-studentt", rows=1024, cols=1024, dtype="f32", tile=128,
            lattices=["E8"], bps=[4.0], seed=0),
    1: dict(name="llama7b-proj-4096x4096-bf16", rows=4096, cols=4096, dtype="bf16", tile=128,
            lattices=["E8"], bps=[4.0], seed=1),
    2: dict(name="llama-mlp-11008x4096-bf16", rows=11008, cols=4096, dtype="bf16", tile=128,
            lattices=["Z", "A2", "D4", "E8"], bps=[3.0, 4.0, 5.0], seed=2),
    3: dict(name="kv-cache-8x32x8192x128-bf16", batch=8, heads=32, seq=8192, head_dim=128,
            dtype="bf16", tile=128, lattices=["E8"], bps=[2.0], seed=3, dither=1),
    4: dict(name="dit-stack-48x4096x16384-bf16", layers=48, rows=4096, cols=16384, dtype="bf16",
            tile=256, lattices=["E8"], bps=[4.0], seed=4),
}


def config_tensor(cfg: int, layer: int = 0, which: str = "K") -> np.ndarray:
    """fp32 numpy array of configuration `cfg` (layer of the DiT stack; K or V of
    the KV cache).  bf16 configurations are rounded by the caller (to_bf16)."""
    c = CONFIGS[cfg]
    if cfg == 0:
        return student_t_outlier_cols(c["rows"], c["cols"], key=0)
    if cfg in (1, 2):
        return gaussian_outlier_channels(c["rows"], c["cols"], key=cfg)
    if cfg == 3:
        return kv_cache(c["batch"], c["heads"], c["seq"], c["head_dim"], key=3, which=which)
    if cfg == 4:
        return dit_layer(c["rows"], c["cols"], key=4, layer=layer)
    raise KeyError(cfg)


def codec_seed(cfg: int, layer: int = 0, which: str = "K") -> int:
    """Codec seed: the config's seed; per DiT layer (4 << 32) | layer; V of the
    KV cache 3 + 2^32 (a different per-layer sign diagonal and dither)."""
    if cfg == 4:
        return (4 << 32) | layer
    if cfg == 3:
        return 3 if which == "K" else 3 + (1 << 32)
    return cfg


def dit_layer_device(rows: int, cols: int, layer: int, device, std: float = 0.02,
                     p_out: float = 0.005, nu: int = 3) -> "torch.Tensor":
    """dit_layer's distribution drawn directly on `device` with torch's
    generator seeded by (4, layer) — the 6.4 GB stack would take minutes to
    draw on the host.  Student-t(nu) = N / sqrt(chi2_nu / nu).  Returns bf16."""
    g = torch.Generator(device=device)
    g.manual_seed((4 << 32) | layer)
    w = std * torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    mask = torch.rand(rows, cols, generator=g, device=device) < p_out
    z = torch.randn(rows, cols, generator=g, device=device)
    chi = torch.zeros(rows, cols, device=device)
    for _ in range(nu):
        e = torch.randn(rows, cols, generator=g, device=device)
        chi += e * e
    t = z / torch.sqrt(chi / nu)
    w = torch.where(mask, t, w)
    return w.to(torch.bfloat16)


def e8_near_ties(n: int, key: int, span: int = 120) -> np.ndarray:
    """n blocks of 8 fp32 coordinates near the bisector of a point A of D8 and
    a neighbouring point B of D8 + 1/2 (A - B in {+-1/2}^8 with an even count
    of minus signs, |A - B|^2 = 2): t = (A + B)/2 + w, w a random vector
    orthogonal to A - B of length up to 0.1, then some coordinates nudged by
    up to 1e-6 of that length; A ranges over |coordinates| <= 2 span.  A
    quarter of the blocks take w = 0 and no nudge (exact ties in fp32)."""
    rng = _rng(11, key)
    d = 2 * rng.integers(-span // 2, span // 2 + 1, size=(n, 8))
    d[:, 0] += 2 * rng.integers(0, 2, n)
    v = np.where(rng.random((n, 8)) < 0.5, -0.5, 0.5)
    odd = (v < 0).sum(axis=1) % 2 == 1
    v[odd, 0] = -v[odd, 0]
    w = rng.standard_normal((n, 8)) * rng.uniform(0.0, 0.1, (n, 1))
    w -= ((w * v).sum(axis=1, keepdims=True) / 2.0) * v          # |v|^2 = 2
    w += rng.choice([0.0, 1.0, -1.0], size=(n, 8)) * 1e-6 * rng.random((n, 1))
    w[: n // 4] = 0.0
    t = (d + 0.5) + v / 2.0 + w                                   # B = d + 1/2, A = B + v
    return t.astype(np.float32)


def haar_orthogonal(d: int, key: int) -> np.ndarray:
    """A Haar-uniform d x d orthogonal matrix (the KV path's per-layer
    rotation is drawn by the caller): QR of an fp64 Gaussian matrix with the
    signs of R's diagonal moved into Q (Mezzadri's correction), rounded to
    fp32, row-major."""
    g = _rng(7, key).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q, dtype=np.float32)
