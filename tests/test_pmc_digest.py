"""The rocprofv3 digest (kv_cache_tile_amd/pmc_digest.py) on small synthetic
counter and trace files: per-kernel averages over dispatches, the last-N
selection, the copy-kernel scaling of FETCH_SIZE / WRITE_SIZE, and the
kernel-source digest that gates bench.py's use of the summaries."""
import csv
import json
import os

import bench
from kv_cache_tile_amd import pmc_digest as pd

ENC = "void hq::encode_kernel<8, 256, false, true>(void const*, unsigned int)"
DEC = "void hq::decode_kernel<8, 256, false, false>(unsigned int const*)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"


def _counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Correlation_Id", "Dispatch_Id", "Agent_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for did, name, counter, value in rows:
            w.writerow([did, did, 1, name, counter, value])


def test_sq_averages_and_last(tmp_path):
    d = str(tmp_path / "s")
    rows = []
    # encode dispatches 1..4 (VALU 100, 200, 300, 400), decode 5..6; a
    # counter may arrive in several rows per dispatch (summed)
    for i, v in enumerate((100, 200, 300, 400)):
        rows += [(i + 1, ENC, "SQ_INSTS_VALU", v / 2), (i + 1, ENC, "SQ_INSTS_VALU", v / 2),
                 (i + 1, ENC, "SQ_WAVES", 64)]
    rows += [(5, DEC, "SQ_INSTS_VALU", 50), (6, DEC, "SQ_INSTS_VALU", 70), (7, NEG, "SQ_INSTS_VALU", 1e9)]
    _counters(d, rows)
    allk = pd.sq_summary([d], numel=64)
    assert set(allk) == {"encode_kernel", "decode_kernel"}            # library kernels only
    assert allk["encode_kernel"]["valu_insts_per_launch"] == 250.0
    assert allk["encode_kernel"]["valu_per_scalar"] == 250.0          # x 64 lanes / 64 scalars
    assert allk["decode_kernel"]["valu_insts_per_launch"] == 60.0
    last = pd.sq_summary([d], numel=64, last=2)
    assert last["encode_kernel"]["dispatches"] == 2 and last["encode_kernel"]["valu_insts_per_launch"] == 350.0
    assert last["decode_kernel"]["valu_insts_per_launch"] == 60.0


def test_traffic_scaled_by_the_copy(tmp_path):
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    # the copy reads and writes 1 MiB; its FETCH_SIZE reads half of that (factor 2)
    _counters(f, [(1, ENC, "FETCH_SIZE", 100.0), (2, ENC, "FETCH_SIZE", 300.0), (3, NEG, "FETCH_SIZE", 512.0)])
    _counters(w, [(1, ENC, "WRITE_SIZE", 10.0), (2, ENC, "WRITE_SIZE", 30.0), (3, NEG, "WRITE_SIZE", 1024.0)])
    out = str(tmp_path / "t.json")
    pd.main(["traffic", "--fetch", f, "--write", w, "--copy-mib", "1", "--alg", "100000", "--workload", "x",
             "--command", "y", "--out", out])
    rec = json.load(open(out))
    k = rec["kernels"]["encode_kernel"]
    assert rec["copy_reference"]["fetch_scale"] == 2.0 and rec["copy_reference"]["write_scale"] == 1.0
    assert k["hbm_read_bytes"] == 200 * 1024 * 2 and k["hbm_write_bytes"] == 20 * 1024
    assert rec["kernel_source_sha256"] == bench.kernel_source_digest()


def test_short_names_and_trace_last(tmp_path, capsys):
    assert pd.short_name(ENC) == "encode_kernel<E8, 256, no dither, bf16 input>"
    assert pd.short_name(DEC) == "decode_kernel<E8, 256, no dither>"
    assert pd.short_name("void hq::decode_kernel<4, 128, true, false>(x)") == "decode_kernel<D4, 128, dither>"
    d = tmp_path / "k"
    d.mkdir()
    with open(d / "k_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, dur in enumerate((9000, 1000, 3000, 5000)):          # ns
            w.writerow([i + 1, ENC, 10_000 * i, 10_000 * i + dur])
    pd.main(["trace", "--dir", str(d), "--last", "2"])
    out = capsys.readouterr().out
    assert "| `encode_kernel<E8, 256, no dither, bf16 input>` | 2 | 4.0 | 3.0 | 5.0 |" in out


def test_bench_reads_counters_only_for_current_sources(tmp_path, monkeypatch):
    rec = {"kernel_source_sha256": bench.kernel_source_digest(),
           "kernels": {"encode_kernel": {"valu_insts_per_launch": 1.0e6}}}
    p = tmp_path / "c.json"
    p.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(p))
    assert bench.measured_valu("encode_kernel") == 1.0e6
    r = bench.roofline("encode_kernel", 10.0, 1.0e6, 1 << 20)
    assert r["bound"] in ("alu", "hbm") and "valu_per_scalar" in (r if r["bound"] == "alu" else r["valu"])
    rec["kernel_source_sha256"] = "0" * 64
    p.write_text(json.dumps(rec))
    assert bench.measured_valu("encode_kernel") is None
    assert bench.roofline("encode_kernel", 10.0, 1.0e6, 1 << 20)["bound_source"] == "no current VALU counters"

