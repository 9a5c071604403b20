"""Host-side logic of bench.py: the per-configuration oracle leg of
`bench.py --configs` (a timed, bit-exact-checked sample of each run's stream),
exercised on streams the oracle writes itself, so no GPU is needed."""
import bench


def test_oracle_leg_checks_the_sample():
    # bench.py's per-configuration oracle leg on streams the oracle itself
    # wrote: whole-chunk samples compare bit-exact, and one flipped bit in
    # the decoded values is reported
    import types

    import numpy as np
    import torch

    import oracle
    from kv_cache_tile_amd import workloads
    for rows, cols, tile, bf16, dither in ((256, 1024, 128, False, 0), (300, 4096, 128, True, 0),
                                           (2048, 128, 128, True, 1)):
        x = workloads.gaussian(rows, cols, key=rows)
        if bf16:
            x = workloads.bf16_bits(workloads.to_bf16(x))
        c, seed = 0.29, 5
        e = oracle.encode(x, tile, "E8", c, seed, dither=dither)
        xo, st = oracle.decode(e, rows, cols, tile, "E8", c, seed, oracle.BF16 if bf16 else oracle.F32, dither=dither)
        assert st == oracle.OK
        h = types.SimpleNamespace(step=torch.from_numpy(e.step.view(np.int16)),
                                  meta=torch.from_numpy(e.meta.view(np.int16)),
                                  chunk_off=torch.from_numpy(e.chunk_off.view(np.int32)),
                                  payload=torch.from_numpy(e.payload.view(np.int32)))
        out = torch.from_numpy(xo.view(np.int16 if bf16 else np.int32).copy())
        out = out.view(torch.bfloat16 if bf16 else torch.float32)
        r = bench.cpu_baseline_config(x, rows, cols, tile, "E8", c, seed, dither, h, out, max_scalars=1 << 17)
        assert r["parity_sample"] == "bit-exact" and r["cores"] == 1
        n = int(r["sample"].split()[1])
        assert n * cols <= max(1 << 17, cols * 64) and (n * (cols // tile)) % 64 == 0 or n == rows
        bad = out.clone()
        bad.view(torch.int16 if bf16 else torch.int32)[0, 0] ^= 1
        assert bench.cpu_baseline_config(x, rows, cols, tile, "E8", c, seed, dither, h, bad,
                                         max_scalars=1 << 17)["parity_sample"].startswith("MISMATCH")
