#!/usr/bin/env python3
"""Benchmark of the GRINQH decode GEMV on one MI355X.

One step = the three 8B-shaped decode linears (4096->4096, 4096->14336,
14336->4096; b_max 8; bf16 x ~ Student-t(3); per-output fp16 s, z; bf16 y)
at about 3 effective bits, as three grinqh_gemv calls one after another (the
order a decoder runs them in: each call is its own kernel launch doing bit
assignment, prefix-plane streaming, midpoint dequant and the product).
Inputs are resident in HBM before timing starts.  Every timed launch
rotates over enough packed weight copies that the plane bytes its linear
reads over one rotation are at least twice the 256 MB Infinity Cache (sized
at the fewest bits timed), so no launch finds its planes there.  The timed
region is one HIP graph holding exactly K steps, bracketed by device
synchronisation and HIP events on the launch stream.

Reported value: required bytes per second, where required bytes = taken
2-bit planes (sum_i b_i * d_out / 8) + fp16 s and z (4 * d_out), summed over
the step's GEMVs.  Also reported, each GEMV in its own launch unless stated:
 * b_max 8 sweep over 2/3/4/8 effective bits (8 = every channel at b_max: the
   dense dequant GEMV of the same kernel), the same three linears as one
   grinqh_gemv_group launch, and a straight-line fit of latency against
   effective bits per linear (intercept = the fixed cost of a launch);
 * b_max 4 (levels 0/2/4) at 1.5/2/3/4 effective bits, 4 being its dense mode;
 * b_max 6 (levels 0/2/4/6) at 2/3/4/6;
 * the 70B shapes (8192->8192, 8192->28672, 28672->8192) at 2 and 3 bits,
   rotating over weight copies sized the same way (about 7 GB of planes);
 * the whole 32-layer 8B decode step (128 launches in dependency order: per
   layer fused q|k|v, o, fused gate|up, down; 7.0 GB of planes at b_max 8) at
   2/3/4/6/8 bits, with its fit;
 * the offline threshold calibration and RTN quantisation, and the prefill
   dense b_max GEMM on the matrix cores (TFLOP/s against the bf16 peak, with
   torch's bf16 matmul of a dense weight of the same shape beside it);
 * the plain fp64 C oracle timed on the host, on one thread and on every
   core, over a bounded sample.

    python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMV µs and required-bytes HBM GB/s (% of MI355X peak) at 2/3/4/8 eff. bits"
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
MAX_COPIES = 256


KERNEL_SOURCES = ("input_adaptive_bit_amd/csrc/gemv.hip", "input_adaptive_bit_amd/csrc/decode.hpp",
                  "input_adaptive_bit_amd/csrc/device_common.hpp", "input_adaptive_bit_amd/csrc/internal.h")
COUNTER_SUMMARY = "profiles/gemv_one_kernel__8b_decode_linears_e3__hbm_counters.md"
SQ_SUMMARY = "profiles/gemv_one_kernel__8b_decode_linears_e3__sq_counters.md"


# What the pages report for this path (GRINQH note, papernotes.org, the
# hardware throughput and ablation table; and the summary page's key
# results), restated: model-level decode throughput on one RTX 4090, not a
# kernel figure and not comparable with this GPU's numbers.
PAGES_CONTEXT = {
    "hardware": "1x NVIDIA RTX 4090 (custom Triton GEMV, 8B model)",
    "decode_tok_per_s": {"GPTQ 4-bit MARLIN": 160.4, "GRINQH b_max 8, 4 eff. bits": 157.6,
                         "GRINQH b_max 8, 3 eff. bits": 182.2, "GRINQH b_max 8, 2 eff. bits": 204.6},
    "claims": ["decode up to 1.28x the tokens/s of 4-bit MARLIN (at 2 effective bits)",
               "latency scaling in proportion to the effective bits"],
    "use": "context only",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def required_bytes(bits_np: np.ndarray, d_out: int) -> float:
    return float(bits_np.astype(np.int64).sum()) * d_out / 8.0 + 4.0 * d_out


def kernel_sources_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_field(path: str, field: str, eff: int):
    """A per-launch figure from a committed counter summary, or None when that
    summary was taken on other kernel sources or another workload."""
    if eff != 3:
        return None
    try:
        with open(os.path.join(ROOT, path)) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_", "kernel_", "valu_")))
    if fields.get("kernel_sources_sha256", "").strip() != kernel_sources_hash():
        return None
    if fields.get("traffic_workload", "").strip() != "per-call" or field not in fields:
        return None
    return float(fields[field])


def counted_traffic(eff: int):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary
    (scaled by a copy kernel of known size), or None (see counted_field)."""
    v = counted_field(COUNTER_SUMMARY, "traffic_bytes_per_launch", eff)
    return None if v is None else int(v)


def fit_line(xs, ys):
    """Least-squares y = a + b x: (a, b)."""
    x = np.asarray(xs, np.float64)
    y = np.asarray(ys, np.float64)
    b, a = np.polyfit(x, y, 1)
    return float(a), float(b)


class Shape:
    """One linear on the device: packed code copies (copy 0 from the numpy
    generator, the rest drawn on the device), s, z, x, and a threshold vector
    per effective-bits target (same codes, scales and x for all).

    n_copies = 0 sizes the rotation by the bytes the launches actually read:
    enough copies that one pass over them reads, at the fewest bits timed,
    at least twice the 256 MB Infinity Cache (and at least 4 copies), so no
    launch can find its planes there."""

    def __init__(self, spec, n_copies, dev, effs, host_codes=True):
        import torch
        import input_adaptive_bit_amd as G
        import synthetic as S
        self.spec = spec
        self.d_in, self.d_out = spec.d_in, spec.d_out
        lin = S.make_linear(spec, with_codes=host_codes)
        self.q0 = lin.q                                  # host codes of copy 0 (CPU baseline)
        self.s_np, self.z_np, self.x_f32 = lin.s, lin.z, lin.x
        self.L = G.grinqh_layout_init(spec.d_in, spec.d_out, spec.b_max)
        self.planes = []
        self._add_copy(dev, lin.q if host_codes else None)
        self.s = torch.from_numpy(lin.s).to(dev)
        self.z = torch.from_numpy(lin.z).to(dev)
        self.x = torch.from_numpy(lin.x_bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        self.ws = G.new_workspace(self.L, dev)
        self.y = torch.empty(spec.d_out, dtype=torch.bfloat16, device=dev)
        self.theta = {}
        self.theta_np = {}
        self.bits = {}
        self.req = {}
        for eff, sp in effs.items():
            th = S.make_linear(sp, with_codes=False).theta
            self.theta_np[eff] = th
            self.theta[eff] = torch.from_numpy(th).to(dev)
            bits, _, _ = G.assign_bits(self.L, self.x, self.theta[eff])
            torch.cuda.synchronize()
            b = bits.cpu().numpy()
            self.bits[eff] = b
            self.req[eff] = required_bytes(b, self.d_out)
        if n_copies <= 0:
            least = min(self.req[e] - 4.0 * self.d_out for e in effs)      # plane bytes read per launch
            n_copies = min(MAX_COPIES, max(4, math.ceil(2 * MALL_BYTES / max(least, 1.0))))
        while len(self.planes) < n_copies:
            self._add_copy(dev, None)
        torch.cuda.synchronize()
        self.n_copies = n_copies

    def _add_copy(self, dev, q_host) -> None:
        import torch
        import input_adaptive_bit_amd as G
        import synthetic as S
        if q_host is not None:
            qd = torch.from_numpy(q_host).to(dev)
        else:
            g = torch.Generator(device=dev)
            g.manual_seed(S.torch_seed(self.spec.key, 10 + len(self.planes)))
            qd = torch.randint(0, 1 << self.spec.b_max, (self.d_out, self.d_in), generator=g, dtype=torch.uint8,
                               device=dev)
        _, pl = G.pack(qd, self.spec.b_max)
        self.planes.append(pl)
        del qd

    def launch(self, copy: int, eff) -> None:
        import input_adaptive_bit_amd as G
        G.grinqh_gemv(self.L, self.x, self.theta[eff], self.planes[copy % self.n_copies], self.s, self.z, self.y,
                      self.ws)

    def operands(self, copy: int, eff):
        return (self.x, self.theta[eff], self.planes[copy % self.n_copies], self.s, self.z, self.y)

    def eff_bits(self, eff) -> float:
        return float(self.bits[eff].astype(np.float64).mean())


class GroupStep:
    """The linears of a step as one grinqh_gemv_group launch."""

    def __init__(self, shapes, dev):
        import input_adaptive_bit_amd as G
        self.shapes = shapes
        self.layouts = [sh.L for sh in shapes]
        self.ws = G.new_group_workspace(self.layouts, dev)

    def launch(self, copy: int, eff) -> None:
        import input_adaptive_bit_amd as G
        G.grinqh_gemv_group(self.layouts, [sh.operands(copy, eff) for sh in self.shapes], self.ws)


class DecodeStep:
    """The whole 32-layer 8B-shaped decode step as decode must launch it: per
    layer the fused q|k|v projection (4096->6144), o (4096->4096), the fused
    gate|up projection (4096->28672) and down (14336->4096), one grinqh_gemv
    launch each, in that order (o and down depend on the launch before them),
    each with its own activations and thresholds; codes drawn on the device
    from seeded generators (7.0 GB of planes at b_max 8)."""

    def __init__(self, dev, effs, n_layers=32, unfused=False):
        import torch
        import input_adaptive_bit_amd as G
        import synthetic as S
        if unfused:
            # the seven linears of a layer as separate launches; q, k and v
            # (and gate and up) read the same x and thresholds
            pairs = S.llama8b_decode_step_unfused(3, n_layers)
        else:
            pairs = [(spec, spec.key) for spec in S.llama8b_decode_step(3, n_layers)]
        self.ops = []
        self.req = {e: 0.0 for e in effs}
        inputs = {}
        for spec, in_key in pairs:
            g = torch.Generator(device=dev)
            g.manual_seed(S.torch_seed(spec.key, 0))
            q = torch.randint(0, 256, (spec.d_out, spec.d_in), generator=g, dtype=torch.uint8, device=dev)
            L, planes = G.pack(q, 8)
            del q
            s_np, z_np = S.gen_scales(spec)
            if in_key not in inputs:
                xs, _ = S.gen_x_stream(spec)
                x = torch.from_numpy(S.f32_to_bf16_bits(xs[spec.n_calib]).view(np.int16).copy()).to(dev)
                inputs[in_key] = (x, {e: torch.from_numpy(S.calibrate_theta(xs[:spec.n_calib], S.QUANTILES_B8[e], 4)).to(dev)
                                      for e in effs})
            x, th = inputs[in_key]
            for e in effs:
                bits, _, _ = G.assign_bits(L, x.view(torch.bfloat16), th[e])
                self.req[e] += required_bytes(bits.cpu().numpy(), spec.d_out)
            self.ops.append(dict(L=L, planes=planes, x=x.view(torch.bfloat16), th=th,
                                 s=torch.from_numpy(s_np).to(dev), z=torch.from_numpy(z_np).to(dev),
                                 y=torch.empty(spec.d_out, dtype=torch.bfloat16, device=dev),
                                 ws=G.new_workspace(L, dev)))
        torch.cuda.synchronize()

    def launch(self, eff) -> None:
        import input_adaptive_bit_amd as G
        for o in self.ops:
            G.grinqh_gemv(o["L"], o["x"], o["th"][eff], o["planes"], o["s"], o["z"], o["y"], o["ws"])


def capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def time_graph(g, reps: int = 1) -> float:
    """Milliseconds for `reps` replays, events on the current stream (the
    stream the library's kernels are launched on)."""
    import torch
    st = torch.cuda.Event(enable_timing=True)
    en = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    st.record()
    for _ in range(reps):
        g.replay()
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en)


def time_per_rep(fn_rep, reps: int) -> float:
    """Microseconds per repetition of fn_rep(r), r = 0 .. reps-1, captured in
    one graph: the median of three replays after one warm replay."""
    g = capture(lambda: [fn_rep(r) for r in range(reps)])
    time_graph(g)
    ts = sorted(time_graph(g) for _ in range(3))
    del g
    return ts[1] * 1e3 / reps


def point(us: float, req: float, **extra) -> dict:
    gbs = req / (us * 1e-6) / 1e9
    return dict({"us": round(us, 3), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                 "required_MB": round(req / 1e6, 3)}, **extra)


def sweep_shapes(shapes, effs, reps, group=None, dense_key=None):
    """Per effective-bits target: each linear in its own launch, the linears
    one after another (the step), and optionally one group launch.  A timed
    graph holds at least one launch per weight copy, so it reads every copy."""
    reps = max(reps, max(sh.n_copies for sh in shapes))
    out = {}
    for e in effs:
        row = {}
        for sh in shapes:
            t = time_per_rep(lambda r, sh=sh, e=e: sh.launch(r, e), reps)
            row[f"{sh.d_in}x{sh.d_out}"] = point(t, sh.req[e], eff_bits=round(sh.eff_bits(e), 4))
        req = sum(sh.req[e] for sh in shapes)
        t = time_per_rep(lambda r, e=e: [sh.launch(r, e) for sh in shapes], reps)
        row["step (one launch per linear)"] = point(t, req)
        if group is not None:
            t = time_per_rep(lambda r, e=e: group.launch(r, e), reps)
            row["step (one group launch)"] = point(t, req)
        key = str(e) if e != dense_key else f"{e} (dense)"
        out[key] = row
        log(f"  eff {key}: " + ", ".join(f"{k} {v['us']} us {v['GB/s']} GB/s" for k, v in row.items()))
    return out


def fits(sweep, shape_keys):
    """Latency against effective bits per linear: intercept (fixed cost of a
    launch), slope, and the marginal bandwidth the slope implies."""
    out = {}
    for k in shape_keys:
        xs = [row[k]["eff_bits"] for row in sweep.values()]
        us = [row[k]["us"] for row in sweep.values()]
        mb = [row[k]["required_MB"] for row in sweep.values()]
        a, b = fit_line(xs, us)
        a_mb, b_mb = fit_line(mb, us)
        out[k] = {"intercept_us": round(a, 3), "us_per_bit": round(b, 3),
                  "marginal_GB/s": round(1e3 / b_mb, 1) if b_mb > 0 else None,
                  "intercept_share_at_3_bits": round(a / (a + 3 * b), 3)}
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_rows():
    """The oracle on bounded samples of the rows after the decode GEMV."""
    import synthetic as S
    rows = {}
    # the prefill oracle (numpy fp64, one BLAS thread) on 8 tokens of the
    # 4096 -> 16384 up projection
    from threadpoolctl import threadpool_limits
    from oracle import grinqh_oracle
    rng = np.random.default_rng(4096)
    q = rng.integers(0, 256, size=(16384, 4096), dtype=np.uint8)
    s_ = rng.uniform(0.001, 0.01, 16384).astype(np.float16)
    z_ = rng.normal(0, 0.01, 16384).astype(np.float16)
    xs = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_normal((8, 4096)).astype(np.float32)))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        grinqh_oracle.prefill_gemm(xs, q, s_, z_, 8)
        el = time.perf_counter() - t0
    rows["prefill"] = {"value": round(8 / el, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                      "TFLOP/s": round(2.0 * 8 * 4096 * 16384 / el / 1e12, 6),
                      "sample": f"8 tokens through 4096->16384 at b_max 8 (numpy fp64 oracle, one thread, {el:.1f} s)"}
    xc = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, 128 * 4096).astype(np.float32)))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        grinqh_oracle.calibrate_thresholds(xc, [0.2, 0.5, 0.8, 0.95])
        el_c = time.perf_counter() - t0
        wq = S.bf16_bits_to_f32(S.f32_to_bf16_bits((rng.standard_normal((4096, 4096)) * 0.02).astype(np.float32)))
        t0 = time.perf_counter()
        grinqh_oracle.quantize_rtn(wq, 8)
        el_r = time.perf_counter() - t0
    rows["threshold_calibration"] = {"value": round(el_c * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
                                    "sample": "128 x 4096 bf16 samples, 4 levels (numpy fp64 oracle, one thread)"}
    rows["rtn_quantisation"] = {"value": round(el_r * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
                               "sample": "4096 x 4096 bf16 weights at b_max 8 (numpy oracle, one thread)"}
    return rows


def _oracle_pass(shapes, eff, threads: int):
    """One pass of the C oracle over the step's linears; with threads > 1 the
    output rows of each linear are split into `threads` contiguous blocks,
    each computed by the unchanged oracle in its own host thread (the C call
    releases the interpreter lock)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import c_oracle
    if threads == 1:
        return [c_oracle.gemv(sh.x_f32, sh.theta_np[eff], sh.q0, sh.s_np, sh.z_np, sh.spec.b_max) for sh in shapes]
    ys = []
    with ThreadPoolExecutor(threads) as ex:
        for sh in shapes:
            edges = np.linspace(0, sh.d_out, threads + 1).astype(int)
            futs = [ex.submit(c_oracle.gemv, sh.x_f32, sh.theta_np[eff], sh.q0[a:b], sh.s_np[a:b], sh.z_np[a:b],
                              sh.spec.b_max) for a, b in zip(edges[:-1], edges[1:])]
            ys.append(np.concatenate([f.result() for f in futs]))
    return ys


def cpu_baseline(shapes, eff, seconds: float, rows: bool = True):
    """The plain fp64 C oracle, as it stands, on whole passes of the step's
    linears: first on one host thread, then on every host core."""
    per_step = sum(sh.req[eff] for sh in shapes)
    cores = os.cpu_count() or 1
    res = {}
    for threads in (1, cores):
        t0 = time.perf_counter()
        passes = 0
        while True:
            _oracle_pass(shapes, eff, threads)
            passes += 1
            el = time.perf_counter() - t0
            if el >= seconds / 2:
                break
        res[threads] = (passes, el)
    p1, e1 = res[1]
    pn, en = res[cores]
    out = {
        "value": round(per_step * pn / en / 1e9, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"{pn} full passes of the 3 linears at ~{eff} eff. bits on {cores} host threads "
                   f"(plain fp64 C oracle, output rows split into {cores} blocks, {en:.1f} s)"),
        "cpu_model": cpu_model(),
        "os_cpu_count": cores,
        "one_thread": {"value": round(per_step * p1 / e1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                       "sample": f"{p1} full passes on one thread ({e1:.1f} s)"},
    }
    if rows:
        out.update(cpu_baseline_rows())
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--eff", type=int, default=3, choices=[2, 3, 4, 8])
    ap.add_argument("--sweep-reps", type=int, default=64, help="launches per sweep point")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-b4", action="store_true", help="skip the b_max 4 sweep")
    ap.add_argument("--no-b6", action="store_true", help="skip the b_max 6 sweep")
    ap.add_argument("--no-70b", action="store_true", help="skip the 70B shapes (4.3 GB of planes)")
    ap.add_argument("--no-decode-step", action="store_true",
                    help="skip the 32-layer decode-step measurement (7.0 GB of planes)")
    ap.add_argument("--decode-effs", default="2,3,4,6,8",
                    help="effective bits of the 32-layer decode step (comma list; the seven-launch form "
                         "runs at those of 3 and 8 listed)")
    ap.add_argument("--no-prefill", action="store_true", help="skip the prefill-stage GEMM timing")
    ap.add_argument("--no-offline", action="store_true", help="skip calibration and RTN timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copies", type=int, default=0,
                    help="weight copies per linear (0: enough that one rotation reads twice the Infinity Cache)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run a plain elementwise fp32 kernel (torch.neg) that reads and "
                         "writes this many MiB, 4 times: the known-size reference for HBM byte counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): this decode GEMV is "
              "built and measured on a single MI355X, and how it would shard across GPUs is a design, not code.",
              flush=True)
        return 2

    import torch
    import input_adaptive_bit_amd as G
    import synthetic as S

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    G.load()
    dev = torch.device("cuda:0")
    effs = (2, 3, 4, 8)
    per_eff_specs = {e: S.llama8b_linears(e) for e in effs}
    shapes = [Shape(per_eff_specs[args.eff][k], args.copies, dev, {e: per_eff_specs[e][k] for e in effs})
              for k in range(3)]
    n_copies = {f"{sh.d_in}x{sh.d_out}": sh.n_copies for sh in shapes}
    log(f"setup: weight copies {n_copies}, "
        f"{sum(sh.n_copies * sh.d_in * sh.d_out for sh in shapes) / 1e9:.2f} GB of planes")
    eff = args.eff

    def steps_fn(n):
        def run():
            for st in range(n):
                for sh in shapes:
                    sh.launch(st, eff)
        return run

    # warmup (eager), then the timed graph of exactly K steps
    steps_fn(2)()
    torch.cuda.synchronize()
    g_warm = capture(steps_fn(max(1, args.warmup))) if args.warmup > 0 else None
    g_timed = capture(steps_fn(args.steps))
    if g_warm is not None:
        time_graph(g_warm)
    torch.cuda.synchronize()
    ms = time_graph(g_timed)
    del g_timed, g_warm
    ms_per_step = ms / args.steps
    step_bytes = sum(sh.req[eff] for sh in shapes)
    value_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    n_launch = 3 * args.steps                  # one kernel launch per linear
    avg_launch_us = ms * 1e3 / n_launch
    bytes_per_launch = step_bytes / 3
    achieved = bytes_per_launch / (avg_launch_us * 1e-6) / 1e9
    eff_real = float(np.sum([sh.bits[eff].astype(np.int64).sum() * sh.d_out for sh in shapes]) /
                     np.sum([sh.d_in * sh.d_out for sh in shapes]))
    log(f"timed: {args.steps} steps in {ms:.3f} ms -> {ms_per_step * 1e3:.2f} us/step, {value_gbs:.1f} GB/s")

    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: 4 x torch.neg over {args.copy_probe_mib} MiB fp32 "
            f"(each reads {args.copy_probe_mib} MiB, writes {args.copy_probe_mib} MiB)")
        del src, dst

    reps = args.sweep_reps
    sweep, sweep_fit = {}, {}
    if not args.no_sweep:
        log("sweep b_max 8:")
        group = GroupStep(shapes, dev)
        sweep = sweep_shapes(shapes, effs, reps, group=group, dense_key=8)
        sweep_fit = fits(sweep, [f"{sh.d_in}x{sh.d_out}" for sh in shapes])
        log(f"  fit: {sweep_fit}")
        del group

    sweep_b4, fit_b4 = {}, {}
    if not args.no_sweep and not args.no_b4:
        effs4 = (1.5, 2, 3, 4)
        specs4 = {e: S.llama8b_linears_b4(e) for e in effs4}
        shapes4 = [Shape(specs4[3][k], 0, dev, {e: specs4[e][k] for e in effs4}, host_codes=False)
                   for k in range(3)]
        log("sweep b_max 4:")
        sweep_b4 = sweep_shapes(shapes4, effs4, reps, dense_key=4)
        fit_b4 = fits(sweep_b4, [f"{sh.d_in}x{sh.d_out}" for sh in shapes4])
        for e, row in sweep_b4.items():
            for sh in shapes4:
                k = f"{sh.d_in}x{sh.d_out}"
                row[k]["vs_dense_us"] = round(row[k]["us"] / sweep_b4["4 (dense)"][k]["us"], 3)
        del shapes4
        torch.cuda.empty_cache()

    sweep_b6 = {}
    if not args.no_sweep and not args.no_b6:
        effs6 = (2, 3, 4, 6)
        specs6 = {e: S.llama8b_linears_b6(e) for e in effs6}
        shapes6 = [Shape(specs6[3][k], 0, dev, {e: specs6[e][k] for e in effs6}, host_codes=False)
                   for k in range(3)]
        log("sweep b_max 6:")
        sweep_b6 = sweep_shapes(shapes6, effs6, reps, dense_key=6)
        del shapes6
        torch.cuda.empty_cache()

    llama70b = {}
    if not args.no_sweep and not args.no_70b:
        effs70 = (2, 3)
        specs70 = {e: S.llama70b_linears(e) for e in effs70}
        shapes70 = [Shape(specs70[3][k], 0, dev, {e: specs70[e][k] for e in effs70}, host_codes=False)
                    for k in range(3)]
        log(f"70B shapes: copies {[sh.n_copies for sh in shapes70]}, "
            f"{sum(sh.n_copies * sh.d_in * sh.d_out for sh in shapes70) / 1e9:.2f} GB of planes")
        llama70b = sweep_shapes(shapes70, effs70, reps)
        del shapes70
        torch.cuda.empty_cache()

    calibration = {}
    rtn = {}
    if not args.no_offline:
        for d_in in (4096, 14336):
            spec = S.LinearSpec(d_in, 4096, 8, "t3", "bf16", S.QUANTILES_B8[3], key=(2, 9, 0, d_in))
            xs, _ = S.gen_x_stream(spec)
            xc = torch.from_numpy(S.f32_to_bf16_bits(xs[:spec.n_calib]).view(np.int16).copy()).to(dev)
            xc = xc.view(torch.bfloat16)
            ws_c = torch.empty(G.grinqh_calibrate_workspace_bytes(), dtype=torch.uint8, device=dev)
            th_c = torch.empty(4, dtype=torch.float32, device=dev)
            lv = list(spec.quantiles)
            t = time_per_rep(lambda r: G.grinqh_calibrate_thresholds(xc, lv, th_c, ws_c), 16)
            calibration[f"{spec.n_calib}x{d_in} bf16"] = {
                "values": int(xc.numel()), "us": round(t, 2), "GB/s": round(xc.numel() * 2 / t / 1e3, 1)}
            log(f"calibration {spec.n_calib}x{d_in}: {t:.1f} us")
        for di, do in S.LLAMA8B_SHAPES:
            gen = torch.Generator(device=dev)
            gen.manual_seed(S.torch_seed((2, 8, di, do), 0))
            wt = (torch.randn((do, di), generator=gen, device=dev) * 0.02).to(torch.bfloat16)
            qt = torch.empty((do, di), dtype=torch.uint8, device=dev)
            st_ = torch.empty(do, dtype=torch.float16, device=dev)
            zt = torch.empty(do, dtype=torch.float16, device=dev)
            t = time_per_rep(lambda r: G.grinqh_quantize_rtn(wt, 8, qt, st_, zt), 8)
            moved = 3.0 * di * do
            rtn[f"{di}x{do}"] = {"us": round(t, 2), "GB/s": round(moved / t / 1e3, 1)}
            del wt, qt
            log(f"rtn {di}x{do}: {t:.1f} us, {moved / t / 1e3:.1f} GB/s")

    prefill = {}
    if not args.no_prefill:
        # prefill stage: a block of prompt tokens through dense b_max weights
        for (M, di, do), bm in (((2048, 4096, 16384), 8), ((2048, 4096, 16384), 4), ((2048, 4096, 4096), 8)):
            gen = torch.Generator(device=dev)
            gen.manual_seed(S.torch_seed((2, 10, di, do), bm))
            qd = torch.randint(0, 1 << bm, (do, di), dtype=torch.uint8, device=dev, generator=gen)
            Lp, pl = G.pack(qd, bm)
            sp = (torch.rand(do, generator=gen, device=dev) * 0.009 + 0.001).half()
            zp = (torch.randn(do, generator=gen, device=dev) * 0.01).half()
            xp = torch.randn((M, di), generator=gen, device=dev).to(torch.bfloat16)
            yp = torch.empty((M, do), dtype=torch.bfloat16, device=dev)
            wsp = torch.empty(G.grinqh_prefill_workspace_bytes(M), dtype=torch.uint8, device=dev)

            def pre(reps=16):
                for _ in range(reps):
                    G.grinqh_prefill_gemm(Lp, xp, pl, sp, zp, yp, wsp)
            g = capture(pre)
            # the clock moves under sustained matrix work: about 80 ms of warm-up
            # replays (the first configuration after the memory-bound sweeps
            # otherwise reads several percent slow), then the median of five
            for _ in range(20):
                time_graph(g)
            t = sorted(time_graph(g) for _ in range(5))[2] * 1e3 / 16
            flops = 2.0 * M * di * do
            # the same product on a dense bf16 weight through torch (hipBLASLt), for context
            wd = torch.randn((do, di), generator=gen, device=dev).to(torch.bfloat16)
            for _ in range(3):
                torch.matmul(xp, wd.t())
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                torch.matmul(xp, wd.t())
            e1.record()
            torch.cuda.synchronize()
            tt = e0.elapsed_time(e1) * 1e3 / 20
            prefill[f"{M}x{di}->{do} b_max {bm}"] = {
                "us": round(t, 2), "TFLOP/s": round(flops / t / 1e6, 1),
                "frac_of_bf16_mfma_peak": round(flops / t / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
                "tokens_per_s": round(M / t * 1e6), "torch_bf16_dense_us": round(tt, 2),
                "torch_bf16_dense_TFLOP/s": round(flops / tt / 1e6, 1), "vs_torch_dense": round(tt / t, 3)}
            del g, qd, pl, xp, yp, wd
            torch.cuda.empty_cache()
            log(f"prefill {M}x{di}->{do} b_max {bm}: {t:.1f} us, {flops / t / 1e6:.1f} TFLOP/s; "
                f"torch bf16 dense {tt:.1f} us")

    decode_step, decode_fit, decode_step_unfused = {}, {}, {}
    if not args.no_decode_step:
        for sh in shapes:
            sh.planes = sh.planes[:1]
            sh.n_copies = 1
        torch.cuda.empty_cache()
        effs_ds = tuple(int(v) for v in args.decode_effs.split(","))
        ds = DecodeStep(dev, list(effs_ds))
        for e in effs_ds:
            t = time_per_rep(lambda r, e=e: ds.launch(e), 4)
            gbs = ds.req[e] / (t * 1e-6) / 1e9
            decode_step[str(e) if e != 8 else "8 (dense)"] = {
                "us": round(t, 2), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "required_GB": round(ds.req[e] / 1e9, 4), "launches": len(ds.ops),
                "us_per_launch": round(t / len(ds.ops), 3)}
            log(f"decode step eff {e}: {t:.1f} us, {gbs:.1f} GB/s")
        if len(effs_ds) >= 2:
            a, b = fit_line([v["required_GB"] for v in decode_step.values()],
                            [v["us"] for v in decode_step.values()])
            decode_fit = {"intercept_us": round(a, 1), "intercept_us_per_launch": round(a / len(ds.ops), 3),
                          "marginal_GB/s": round(1e3 / b, 1) if b > 0 else None}
        del ds
        torch.cuda.empty_cache()
        # the same step with the seven linears of a layer launched one by one
        # (224 launches), as the layer is written; at ~3 bits and dense
        effs_unf = [e for e in (3, 8) if e in effs_ds]
        ds = DecodeStep(dev, effs_unf, unfused=True) if effs_unf else None
        for e in effs_unf:
            t = time_per_rep(lambda r, e=e: ds.launch(e), 4)
            gbs = ds.req[e] / (t * 1e-6) / 1e9
            decode_step_unfused[str(e) if e != 8 else "8 (dense)"] = {
                "us": round(t, 2), "GB/s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
                "required_GB": round(ds.req[e] / 1e9, 4), "launches": len(ds.ops),
                "us_per_launch": round(t / len(ds.ops), 3)}
            log(f"decode step, seven launches per layer, eff {e}: {t:.1f} us, {gbs:.1f} GB/s")
        del ds
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(shapes, eff, args.cpu_seconds, rows=not args.no_prefill)
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": METRIC,
        "value": round(value_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": ("8B-shaped decode linears 4096->4096, 4096->14336, 14336->4096, one grinqh_gemv "
                         f"launch each; b_max 8; ~{eff} eff. bits; batch 1; bf16 x ~ t(3), bf16 y; "
                         "fp16 per-output s, z"),
            "global_batch": 1,
            "seq_len": 1,
            "eff_bits_realized": round(eff_real, 4),
            "weight_copies": n_copies,
            "required_bytes_per_step": int(step_bytes),
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counted_traffic(eff),
            # share of the dispatch's SIMD cycles issuing VALU work (SQ counters; None as for traffic)
            "valu_issue_share": counted_field(SQ_SUMMARY, "valu_issue_share_per_launch", eff),
            "kernel": "gemv_one_kernel (three grinqh_gemv launches per step; per-launch average)",
            "avg_launch_us": round(avg_launch_us, 3),
            "bytes_per_launch": int(bytes_per_launch),
        },
        "cpu_baseline": cpu,
        "sweep": sweep,
        "sweep_fit_us_vs_eff_bits": sweep_fit,
        "sweep_b_max_4": sweep_b4,
        "sweep_b_max_4_fit": fit_b4,
        "sweep_b_max_6": sweep_b6,
        "llama70b_shapes": llama70b,
        "threshold_calibration": calibration,
        "rtn_quantisation_b_max_8": rtn,
        "decode_step_32_layers": decode_step,
        "decode_step_fit_us_vs_GB": decode_fit,
        "decode_step_32_layers_seven_launches_per_layer": decode_step_unfused,
        "pages_context": PAGES_CONTEXT,
        "prefill_gemm": prefill,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
