"""Host-side checks of bench.py's contract (no GPU needed)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for an unsupported run


def test_traffic_lookup_needs_a_counter_row():
    import bench
    assert bench.measured_traffic("hsa_attn", "no-such-workload") is None
    assert bench.measured_traffic("no_such_kernel", "llama8b-layer-s32k-c16") is None


def test_counter_table_rows_are_well_formed():
    """Every row of the committed counter table names a kernel, a workload,
    positive byte counts and the source file and hash it was taken with."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.md")
    rows = []
    for line in open(path):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) == 8 and cells[2].isdigit():
            rows.append(cells)
    assert rows
    for kernel, workload, dispatches, rd, wr, tot, src, h in rows:
        assert int(dispatches) > 0
        assert float(rd) >= 0 and float(wr) >= 0
        assert abs(float(rd) + float(wr) - float(tot)) < 2e-3
        assert src.endswith(".hip") and len(h) == 12
        json.dumps([kernel, workload])      # plain strings
