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


def test_oracle_pass_on_all_cores_matches_one_thread():
    """The all-cores CPU baseline splits each linear's output rows over host
    threads running the unchanged C oracle; the outputs equal one thread's."""
    import types
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    import synthetic as S
    shapes = []
    for di, do in ((300, 1000), (64, 65)):
        spec = S.LinearSpec(di, do, 8, "t3", "bf16", S.QUANTILES_B8[3], key=(9, di, do, 0))
        lin = S.make_linear(spec)
        shapes.append(types.SimpleNamespace(x_f32=lin.x, theta_np={3: lin.theta}, q0=lin.q, s_np=lin.s, z_np=lin.z,
                                            spec=spec, d_out=do))
    one = bench._oracle_pass(shapes, 3, 1)
    many = bench._oracle_pass(shapes, 3, 5)
    for a, b in zip(one, many):
        assert np.array_equal(a, b)


def test_fit_line_recovers_a_line():
    sys.path.insert(0, ROOT)
    import bench
    a, b = bench.fit_line([2, 3, 4, 8], [10.0 + 2 * 1.5, 10.0 + 3 * 1.5, 10.0 + 4 * 1.5, 10.0 + 8 * 1.5])
    assert abs(a - 10.0) < 1e-9 and abs(b - 1.5) < 1e-9


def test_committed_counter_summaries_match_the_kernel_sources():
    """The HBM and SQ counter summaries under profiles/ were taken on the
    kernel sources as they stand (their recorded sha256 matches), so the
    bench line carries their traffic and VALU figures instead of null."""
    sys.path.insert(0, ROOT)
    import bench
    traffic = bench.counted_traffic(3)
    share = bench.counted_field(bench.SQ_SUMMARY, "valu_issue_share_per_launch", 3)
    assert traffic is not None and share is not None
    # the counted traffic is the required bytes plus the split-K adds: close to 1x
    assert 1.0 <= traffic / (50214912 / 3) < 1.2
    assert 0.0 < share < 1.0
    assert bench.counted_traffic(8) is None


def test_every_gemv_profile_was_taken_on_the_current_kernel_sources():
    """Every committed GEMV profile summary names the sha256 of the kernel
    sources it was taken on, and that is the hash of the sources as they
    stand: a kernel change without a new profile fails here."""
    import glob
    import re
    sys.path.insert(0, ROOT)
    import bench
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "gemv_one_kernel__*.md")))
    assert len(files) >= 4
    for f in files:
        with open(f) as fh:
            m = re.search(r"sha256:?\s*([0-9a-f]{64})", fh.read())
        assert m is not None, f
        assert m.group(1) == bench.kernel_sources_hash(), f
