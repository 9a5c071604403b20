"""Benchmark of the HyperQuant encode/decode hot path on one MI355X.

Workload (default): the DiT-scale layer stack — 48 linear weights of
4096 x 16384 bf16 (N(0, 0.02^2) with 0.5% unit-scale Student-t(3) entries),
E8 lattice at 4 bits per scalar, RHT tile 256.  One step = stream-encode all
48 layers, then decode all 48 (the whole hot path).  Inputs, outputs and
compressed buffers are resident in HBM before the timed region.

Prints ONE JSON line.  `value` = GB/s of bf16 input through a full round
trip (encode + decode); encode and decode rates are reported separately,
with the fraction of the 8 TB/s HBM peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "encode/decode GB/s of bf16 input (E8, 4 bps) at 1 GPU; % of HBM peak"
KERNEL_SOURCES = ("kv_cache_tile_amd/csrc/hq_lib.hip", "kv_cache_tile_amd/csrc/hq_kernels.h",
                  "kv_cache_tile_amd/csrc/hq_device.h", "kv_cache_tile_amd/csrc/hq_kern_e8.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dit_stack_e8_4bps_hbm_traffic.json")


def kernel_source_digest() -> str:
    """sha256 over the kernel sources: HBM traffic measured with the counters
    is only reported while the kernels are the ones it was measured on."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for
    a plain copy of known size), or None if absent or stale."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def algorithmic_bytes(numel: int, tiles: int, chunks: int, bps: float) -> float:
    """Bytes one encode (or decode) launch must move: the bf16 tensor (2 B per
    scalar), the payload at the target rate (bps/8 B per scalar), step + meta
    (4 B per tile) and the chunk offsets (4 B per chunk)."""
    return numel * (2.0 + bps / 8.0) + 4.0 * tiles + 4.0 * (chunks + 1)


def cpu_baseline(layers_host, rows, cols, tile, bps, seed_of, c):
    """The oracle as it stands, single-threaded on this host, on a bounded
    sample: encode + decode of the given layers."""
    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle
    oracle.build(force=False)
    t_enc = t_dec = 0.0
    n = 0
    for li, xb in layers_host:
        t0 = time.perf_counter()
        e = oracle.encode(xb, tile, "E8", c, seed_of(li))
        t1 = time.perf_counter()
        oracle.decode(e, rows, cols, tile, "E8", c, seed_of(li), oracle.BF16)
        t2 = time.perf_counter()
        t_enc += t1 - t0
        t_dec += t2 - t1
        n += xb.size
    gb = 2.0 * n / 1e9
    return {"value": round(gb / (t_enc + t_dec), 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(layers_host)} of 48 layers ({n} scalars), encode {gb / t_enc:.4f} GB/s, "
                      f"decode {gb / t_dec:.4f} GB/s, {t_enc + t_dec:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--layers", type=int, default=48)
    ap.add_argument("--cpu-layers", type=int, default=2, help="layers timed on the CPU oracle (0 = skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after the timed steps, run one plain copy kernel over this many MiB "
                         "(reference point for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); the codec "
              f"shards by layer or row slab with no communication, see DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from kv_cache_tile_amd import hq, workloads

    dev = torch.device("cuda:0")
    L, rows, cols, tile, lat, bps = args.layers, 4096, 16384, 256, "E8", 4.0
    seed_of = lambda l: (4 << 32) | l  # noqa: E731
    p = hq.plan(hq.BF16, rows, cols, tile, lat, bps)
    xs = [workloads.dit_layer_device(rows, cols, l, dev) for l in range(L)]
    hs = [hq.encode(xs[l], tile, lat, bps, seed_of(l)) for l in range(L)]
    outs = [torch.empty_like(xs[0]) for _ in range(L)]
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(2 * L)]

    def step(record: bool):
        for l in range(L):
            if record:
                ev[l][0].record(stream)
            hq.encode(xs[l], tile, lat, bps, seed_of(l), out=hs[l], zero_status=False)
            if record:
                ev[l][1].record(stream)
        for l in range(L):
            if record:
                ev[L + l][0].record(stream)
            hq.decode(hs[l], out=outs[l])
            if record:
                ev[L + l][1].record(stream)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    enc_ms, dec_ms = [], []
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
        torch.cuda.synchronize()
        enc_ms += [ev[l][0].elapsed_time(ev[l][1]) for l in range(L)]
        dec_ms += [ev[L + l][0].elapsed_time(ev[L + l][1]) for l in range(L)]
    wall = time.perf_counter() - t0
    ms_per_step = 1000.0 * wall / args.steps
    if args.calib_copy_mib > 0:
        # reads and writes exactly calib_copy_mib MiB (int32 negation kernel)
        src = torch.ones(args.calib_copy_mib << 18, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    flags = sum(h.flags() for h in hs)
    bits_payload = sum(h.bits_payload() for h in hs)
    bits_total = sum(h.bits_total() for h in hs)
    numel = rows * cols
    err = sum(float(((o.float() - x.float()) ** 2).sum()) for o, x in zip(outs, xs))
    ref = sum(float((x.float() ** 2).sum()) for x in xs)

    in_gb = 2.0 * numel * L / 1e9
    enc_s = sum(enc_ms) / args.steps / 1000.0
    dec_s = sum(dec_ms) / args.steps / 1000.0
    enc_gbps, dec_gbps = in_gb / enc_s, in_gb / dec_s
    value = in_gb / (enc_s + dec_s)
    alg = algorithmic_bytes(numel, p.tiles, p.chunks, bps)
    enc_avg_us = 1000.0 * sum(enc_ms) / len(enc_ms)
    dec_avg_us = 1000.0 * sum(dec_ms) / len(dec_ms)
    dom_name, dom_us = ("encode_kernel", enc_avg_us) if enc_avg_us >= dec_avg_us else ("decode_kernel", dec_avg_us)
    achieved = alg / (dom_us * 1e-6) / 1e9

    cpu = None
    if args.cpu_layers > 0:
        host = [(l, workloads.bf16_bits(xs[l])) for l in range(min(args.cpu_layers, L))]
        cpu = cpu_baseline(host, rows, cols, tile, bps, seed_of, p.rate_constant)

    rec = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"dit-stack-{L}x{rows}x{cols}-bf16", "lattice": lat, "bps": bps,
                   "tile": tile, "layers": L, "round_trip": "encode all layers, then decode all layers"},
        "encode_GBps": round(enc_gbps, 2), "decode_GBps": round(dec_gbps, 2),
        "encode_hbm_frac_input": round(enc_gbps / HBM_PEAK_GBPS, 4),
        "decode_hbm_frac_input": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "encode_us_per_layer": round(enc_avg_us, 2), "decode_us_per_layer": round(dec_avg_us, 2),
        "bps_payload": round(bits_payload / (numel * L), 4), "bps_total": round(bits_total / (numel * L), 4),
        "compression_vs_bf16": round(16.0 * numel * L / bits_total, 3), "nmse": err / ref, "status_flags": flags,
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom_name), "algorithmic_bytes_per_launch": alg,
                     "avg_launch_us": round(dom_us, 2)},
        "roofline_per_kernel": {
            nm: {"achieved": round(alg / (us * 1e-6) / 1e9, 1), "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                 "avg_launch_us": round(us, 2), "traffic": measured_traffic(nm)}
            for nm, us in (("encode_kernel", enc_avg_us), ("decode_kernel", dec_avg_us))},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
