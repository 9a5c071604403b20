"""HyperQuant encode/decode hot path for MI355X (gfx950): a C-ABI HIP library
(libhq.so, see include/hq.h) with a thin Python binding.

    from kv_cache_tile_amd import hq
    h = hq.encode(w_bf16_cuda, tile=128, lattice="E8", bps=4.0, seed=0)
    w_hat = hq.decode(h)
    k = hq.kv_encode(k_cache, lattice="E8", bps=2.0, seed=layer_seed)
"""
__all__ = ["hq", "workloads", "build"]
