"""Small helpers shared by the tests (no codec arithmetic here)."""
import json
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
RATE_TABLE = os.path.join(ROOT, "kv_cache_tile_amd", "rate_table.json")

_table = None


def rate_c(lattice: str, tile: int, bps: float, dither: int = 0) -> float:
    """Rate constant from the frozen table written by oracle/calibrate.py."""
    global _table
    if _table is None:
        _table = json.load(open(RATE_TABLE))
    for e in _table["entries"]:
        if e["lattice"] == lattice and e["tile"] == tile and e["dither"] == dither and e["bps"] == bps:
            return float(np.array([int(e["c_bits"], 16)], np.uint32).view(np.float32)[0])
    raise KeyError((lattice, tile, bps, dither))


def golden_json(name: str):
    return json.load(open(os.path.join(GOLDEN, name)))


def golden_hadamard():
    mats, cur, rows = {}, None, []
    for line in open(os.path.join(GOLDEN, "hadamard_sylvester.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("n="):
            if cur:
                mats[cur] = np.array(rows, np.float64)
            cur, rows = int(line[2:]), []
        else:
            rows.append([float(v) for v in line.split()])
    mats[cur] = np.array(rows, np.float64)
    return mats
