"""Host-side checks of bench.py that need no GPU: the refusal of more than one
GPU, and the oracle timings of the CPU-baseline leg (bounded samples)."""

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr) or "1 GPU" in (r.stdout + r.stderr)


def test_cpu_baseline_rows_report_the_oracle():
    sys.path.insert(0, ROOT)
    import bench
    rows = bench.cpu_baseline_rows()
    assert set(rows) == {"prefill", "threshold_calibration", "rtn_quantisation"}
    for v in rows.values():
        assert v["kind"] == "oracle" and v["cores"] == 1 and v["value"] > 0
    json.dumps(rows)
