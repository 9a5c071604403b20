"""Digest of rocprofv3 counter collections into the summaries under profiles/.

rocprofv3 --pmc ... --output-format csv writes one row per (dispatch,
counter).  This module averages each counter over the dispatches of each
kernel and writes the JSON that bench.py reads (gated on a digest of the
kernel sources), plus a markdown table on stdout.

  python -m kv_cache_tile_amd.pmc_digest sq --run DIR [--run DIR ...] \\
      --numel N --workload TEXT --command TEXT --out FILE.json
      SQ_* / GRBM_* counters: per kernel and launch, VALU, SALU and LDS
      instructions (wave instructions; x 64 per scalar), LDS bank-conflict
      cycles, waves.
  python -m kv_cache_tile_amd.pmc_digest traffic --fetch DIR --write DIR \\
      --copy-mib M --alg BYTES --workload TEXT --command TEXT --out FILE.json
      FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
      same counter reads for a plain copy kernel that reads and writes M MiB
      (the last dispatch whose name matches --copy-pattern).
  python -m kv_cache_tile_amd.pmc_digest table --run LABEL=DIR ... --numel LABEL=N ...
      one markdown row per (label, kernel) from SQ runs, for per-configuration
      tables.
  python -m kv_cache_tile_amd.pmc_digest trace --dir DIR [--last N]
      the kernel-trace statistics (rocprofv3 --kernel-trace --stats) as a
      markdown table; with --last, each library kernel's last N dispatches
      from the per-dispatch trace.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the sources of the encode and decode kernels: counters taken on other sources are stale
KERNEL_SOURCES = ("kv_cache_tile_amd/csrc/hq_lib.hip", "kv_cache_tile_amd/csrc/hq_kernels.h",
                  "kv_cache_tile_amd/csrc/hq_device.h", "kv_cache_tile_amd/csrc/hq_kern_e8.hip")
VALU_PEAK = 256 * 4 * 16 * 2.4e9     # lane-instructions/s: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_key(name: str) -> str:
    """hq::encode_kernel<8, 256, false, true>(...) -> encode_kernel; other
    kernels keep their demangled name up to the first '(' or '<'."""
    m = re.search(r"hq::(\w+)", name)
    if m:
        return m.group(1)
    return re.split(r"[(<]", name.strip(), 1)[0].split()[-1] if name.strip() else name


def read_rows(d: str):
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    rows = []
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                rows.append({k.strip().lower(): v for k, v in r.items() if k is not None})
    return rows


def per_dispatch(rows):
    """{dispatch id: (kernel name, {counter: value})}, in dispatch order."""
    out = {}
    for r in rows:
        did = int(r.get("dispatch_id") or r.get("correlation_id"))
        name = r.get("kernel_name", "")
        c = r["counter_name"]
        v = float(r["counter_value"])
        ent = out.setdefault(did, (name, {}))
        ent[1][c] = ent[1].get(c, 0.0) + v
    return dict(sorted(out.items()))


def averages(dispatches, pattern=None, last=0):
    """{kernel key: {"dispatches": n, counter: mean per dispatch}}, over
    each kernel's last `last` dispatches (0: all)"""
    if last:
        keep, seen = set(), {}
        for did, (name, _) in reversed(list(dispatches.items())):
            k = kernel_key(name)
            if seen.get(k, 0) < last:
                seen[k] = seen.get(k, 0) + 1
                keep.add(did)
        dispatches = {d: v for d, v in dispatches.items() if d in keep}
    acc = {}
    for _, (name, cs) in dispatches.items():
        if pattern and not re.search(pattern, name):
            continue
        k = kernel_key(name)
        a = acc.setdefault(k, {"dispatches": 0, "name": name, "sums": {}})
        a["dispatches"] += 1
        for c, v in cs.items():
            a["sums"][c] = a["sums"].get(c, 0.0) + v
    return {k: {"dispatches": a["dispatches"], "name": a["name"],
                **{c: v / a["dispatches"] for c, v in a["sums"].items()}} for k, a in acc.items()}


def sq_summary(dirs, numel, last=0):
    d = {}
    for dd in dirs:
        d.update({(dd, k): v for k, v in per_dispatch(read_rows(dd)).items()})
    avg = averages({i: v for i, v in enumerate(d.values())}, r"hq::", last)
    out = {}
    for k, a in avg.items():
        rec = {"dispatches": a["dispatches"], "kernel_name": a["name"]}
        for c, field in (("SQ_INSTS_VALU", "valu_insts_per_launch"), ("SQ_INSTS_SALU", "salu_insts_per_launch"),
                         ("SQ_INSTS_LDS", "lds_insts_per_launch"), ("SQ_WAVES", "waves_per_launch"),
                         ("SQ_LDS_BANK_CONFLICT", "lds_bank_conflict_cycles_per_launch"),
                         ("SQ_ACTIVE_INST_VALU", "active_inst_valu_per_launch"),
                         ("SQ_BUSY_CYCLES", "sq_busy_cycles_per_launch"),
                         ("GRBM_GUI_ACTIVE", "gui_active_cycles_per_launch")):
            if c in a:
                rec[field] = round(a[c], 1)
        if "SQ_INSTS_VALU" in a and numel:
            rec["valu_per_scalar"] = round(64.0 * a["SQ_INSTS_VALU"] / numel, 2)
            rec["valu_roof_us"] = round(64.0 * a["SQ_INSTS_VALU"] / VALU_PEAK * 1e6, 2)
        if "SQ_INSTS_SALU" in a and numel:
            rec["salu_per_scalar"] = round(64.0 * a["SQ_INSTS_SALU"] / numel, 2)
        if "SQ_INSTS_LDS" in a and numel:
            rec["lds_per_scalar"] = round(64.0 * a["SQ_INSTS_LDS"] / numel, 3)
        out[k] = rec
    return out


def cmd_sq(args):
    ks = sq_summary(args.run, args.numel, args.last)
    rec = {"workload": args.workload, "command": args.command, "numel": args.numel, "last_dispatches": args.last,
           "kernel_source_sha256": kernel_source_digest(), "kernels": ks}
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print("| kernel | dispatches | waves | VALU / scalar | SALU / scalar | LDS / scalar | LDS bank-conflict cycles "
          "| VALU-roof us |")
    print("|---|---|---|---|---|---|---|---|")
    for k, r in sorted(ks.items()):
        print(f"| `{k}` | {r['dispatches']} | {r.get('waves_per_launch', '')} | {r.get('valu_per_scalar', '')} | "
              f"{r.get('salu_per_scalar', '')} | {r.get('lds_per_scalar', '')} | "
              f"{r.get('lds_bank_conflict_cycles_per_launch', '')} | {r.get('valu_roof_us', '')} |")


def cmd_traffic(args):
    fd, wd = per_dispatch(read_rows(args.fetch)), per_dispatch(read_rows(args.write))

    def copy_reading(d, counter):
        hits = [cs[counter] for _, (name, cs) in d.items() if re.search(args.copy_pattern, name) and counter in cs]
        if not hits:
            raise SystemExit(f"no dispatch matching {args.copy_pattern!r} with {counter}")
        return hits[-1]

    mib_kib = args.copy_mib * 1024.0
    fk, wk = copy_reading(fd, "FETCH_SIZE"), copy_reading(wd, "WRITE_SIZE")
    fs, ws = mib_kib / fk, mib_kib / wk
    fa, wa = averages(fd, r"hq::", args.last), averages(wd, r"hq::", args.last)
    ks = {}
    for k in sorted(set(fa) & set(wa)):
        rb = fa[k]["FETCH_SIZE"] * 1024.0 * fs
        wb = wa[k]["WRITE_SIZE"] * 1024.0 * ws
        ks[k] = {"dispatches_fetch": fa[k]["dispatches"], "dispatches_write": wa[k]["dispatches"],
                 "fetch_kib": round(fa[k]["FETCH_SIZE"], 1), "write_kib": round(wa[k]["WRITE_SIZE"], 1),
                 "hbm_read_bytes": int(rb), "hbm_write_bytes": int(wb), "hbm_bytes_per_launch": int(rb + wb),
                 "algorithmic_bytes_per_launch": args.alg, "ratio_to_algorithmic": round((rb + wb) / args.alg, 4)}
    rec = {"workload": args.workload, "command": args.command, "last_dispatches": args.last,
           "kernel_source_sha256": kernel_source_digest(),
           "copy_reference": {"kernel": f"dispatch matching {args.copy_pattern!r}, {args.copy_mib} MiB read + "
                                        f"{args.copy_mib} MiB written",
                              "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
                              "fetch_scale": round(fs, 5), "write_scale": round(ws, 5)},
           "kernels": ks}
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"fetch factor {fs:.4f} (copy read {fk:.1f} KiB for {mib_kib:.0f}), write factor {ws:.4f}")
    print("| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (scaled) | HBM write MB | total MB "
          "| algorithmic MB | total / algorithmic |")
    print("|---|---|---|---|---|---|---|---|---|")
    for k, r in ks.items():
        print(f"| `{k}` | {r['dispatches_fetch']} / {r['dispatches_write']} | {r['fetch_kib']} | {r['write_kib']} | "
              f"{r['hbm_read_bytes'] / 1e6:.1f} | {r['hbm_write_bytes'] / 1e6:.1f} | "
              f"{r['hbm_bytes_per_launch'] / 1e6:.1f} | {args.alg / 1e6:.1f} | {r['ratio_to_algorithmic']:.3f} |")


def cmd_table(args):
    numel = dict(kv.split("=", 1) for kv in args.numel)
    print("| run | kernel | dispatches | VALU / scalar | SALU / scalar | LDS / scalar | LDS bank-conflict cycles "
          "per launch | VALU-roof us |")
    print("|---|---|---|---|---|---|---|---|")
    for item in args.run:
        label, d = item.split("=", 1)
        ks = sq_summary([d], int(numel[label]))
        for k, r in sorted(ks.items()):
            print(f"| {label} | `{k}` | {r['dispatches']} | {r.get('valu_per_scalar', '')} | "
                  f"{r.get('salu_per_scalar', '')} | {r.get('lds_per_scalar', '')} | "
                  f"{r.get('lds_bank_conflict_cycles_per_launch', '')} | {r.get('valu_roof_us', '')} |")


def short_name(name: str) -> str:
    """hq::encode_kernel<8, 256, false, true>(...) -> encode_kernel<E8, 256, no dither, bf16 input>;
    other kernels: the demangled name up to its argument list, cut to 70 characters."""
    lat = {"1": "Z", "2": "A2", "4": "D4", "8": "E8"}
    m = re.search(r"hq::(encode_kernel|decode_kernel|fused_product_kernel|nearest_kernel)<([^>]*)>", name)
    if m:
        a = [x.strip() for x in m.group(2).split(",")]
        parts = [lat.get(a[0], a[0])] + a[1:2]
        if m.group(1) == "encode_kernel" and len(a) >= 4:
            parts += ["dither" if a[2] == "true" else "no dither", "bf16 input" if a[3] == "true" else "fp32 input"]
        elif m.group(1) == "decode_kernel" and len(a) >= 3:
            parts += ["dither" if a[2] == "true" else "no dither"] + (["int8 codes"] if len(a) > 3 and a[3] == "true" else [])
        return f"{m.group(1)}<{', '.join(parts)}>"
    m = re.search(r"hq::(\w+)", name)
    if m:
        return m.group(1) + (re.search(r"<[^>]*>", name[m.end():]) or [""])[0] if "<" in name[m.end():m.end() + 1] else m.group(1)
    base = name.replace("(anonymous namespace)::", "").split("(")[0]
    base = re.sub(r"^void\s+", "", base)
    base = re.sub(r"^(at::native::|\(anonymous namespace\)::)+", "", base)
    return base[:70]


def cmd_trace_last(args):
    """per kernel (short name), over its last `last` dispatches in the kernel
    trace: calls, average, min and max duration"""
    files = sorted(glob.glob(os.path.join(args.dir, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {args.dir}")
    per = {}
    for fn in files:
        with open(fn, newline="") as f:
            for r in csv.DictReader(f):
                d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                per.setdefault(short_name(r["Kernel_Name"]), []).append((int(r["Dispatch_Id"]), d))
    print(f"| kernel | calls (last) | average us | min us | max us |")
    print("|---|---|---|---|---|")
    for k, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1][-args.last:])):
        if not re.search(args.pattern, k):
            continue
        v = [d for _, d in sorted(v)][-args.last:]
        print(f"| `{k}` | {len(v)} | {sum(v) / len(v) / 1000:.1f} | {min(v) / 1000:.1f} | {max(v) / 1000:.1f} |")


def cmd_trace(args):
    if args.last:
        return cmd_trace_last(args)
    files = sorted(glob.glob(os.path.join(args.dir, "**", "*kernel_stats.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {args.dir}")
    rows = []
    with open(files[0], newline="") as f:
        for r in csv.DictReader(f):
            rows.append({k.strip().lower(): v for k, v in r.items() if k is not None})
    rows.sort(key=lambda r: -float(r.get("totaldurationns", 0)))
    print("| kernel | calls | average us | min us | max us | % of GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows[:args.top]:
        print(f"| `{short_name(r['name'])}` | {r['calls']} | {float(r['averagens']) / 1000:.1f} | "
              f"{float(r['minns']) / 1000:.1f} | {float(r['maxns']) / 1000:.1f} | {float(r['percentage']):.1f} |")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    a = sub.add_parser("sq")
    a.add_argument("--run", action="append", required=True)
    a.add_argument("--numel", type=int, required=True)
    a.add_argument("--workload", required=True)
    a.add_argument("--command", required=True)
    a.add_argument("--out", required=True)
    a.add_argument("--last", type=int, default=0, help="each kernel's last N dispatches only (0: all)")
    b = sub.add_parser("traffic")
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--copy-mib", type=float, required=True)
    b.add_argument("--copy-pattern", default=r"neg")
    b.add_argument("--alg", type=float, required=True)
    b.add_argument("--workload", required=True)
    b.add_argument("--command", required=True)
    b.add_argument("--out", required=True)
    b.add_argument("--last", type=int, default=0, help="each kernel's last N dispatches only (0: all)")
    c = sub.add_parser("table")
    c.add_argument("--run", action="append", required=True)
    c.add_argument("--numel", action="append", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--dir", required=True)
    t.add_argument("--top", type=int, default=12)
    t.add_argument("--last", type=int, default=0, help="each kernel's last N dispatches, from the per-dispatch trace")
    t.add_argument("--pattern", default=r"hq|encode|decode|fused|act_quant|codes_|rotate|nearest",
                   help="with --last: kernels whose short name matches")
    args = ap.parse_args(argv)
    {"sq": cmd_sq, "traffic": cmd_traffic, "table": cmd_table, "trace": cmd_trace}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
