"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bit-exact: packed planes, b_i, the ascending active list and its length,
the decoded codes.  Within tolerance (max relative error, denominator
max(|y*_j|, 1e-2 * rms(y*))): fp32 y <= 2e-3; bf16 y <= 2e-3 + 2^-8 and, for
every output, the fp32 result rounded to nearest even (either neighbour only
within the fp32 results' call-to-call spread of a rounding boundary).  Oracle inputs are the seeded
synthetic arrays; no expected value comes from the HIP path.
"""

import itertools

import numpy as np
import pytest

from oracle import grinqh_oracle as O
from oracle import c_oracle as C
import synthetic as S
from tests.gpu_util import TOL_BF16, TOL_F32, DeviceLinear, require_gpu, say, to_dev, to_dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import input_adaptive_bit_amd as G
    G.load()
    return require_gpu()


@pytest.fixture
def forced_shape():
    """Force a GEMV launch shape for one test; back to automatic afterwards."""
    import input_adaptive_bit_amd as G
    yield G.force_launch_shape
    G.force_launch_shape(0, 0)


def _theta_dev(theta, dev):
    return to_dev(np.asarray(theta, np.float32), dev)


def _mismatch(got, ref, n=8):
    """The outputs that differ most from the oracle: (index, got, ref)."""
    got = np.asarray(got, np.float64)
    d = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-2 * np.sqrt(np.mean(ref ** 2)))
    idx = np.argsort(-d)[:n]
    return [(int(j), float(got[j]), float(ref[j])) for j in idx]


def _check_y(y_dev, y_ref, tol, what):
    import torch
    y = y_dev.float().cpu().numpy().astype(np.float64)
    err = O.max_rel_error(y, y_ref)
    say(f"  {what}: max rel err {err:.3e}")
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.3e}"
    return y


def _run_and_check(dl, x_f32, x_dtype, theta, y_ref, what, dev, check_bf16=True):
    import torch
    xd = to_dev_x(x_f32, x_dtype, dev)
    td = _theta_dev(theta, dev)
    y32 = dl.gemv(xd, td, torch.float32)
    y32b = dl.gemv(xd, td, torch.float32)
    torch.cuda.synchronize()
    y = _check_y(y32, y_ref, TOL_F32, what + " fp32")
    # a second call (workspace reused, slices combined in another order) agrees
    # to fp32 rounding
    y2 = y32b.cpu().numpy().astype(np.float64)
    assert O.max_rel_error(y2, y) <= 5e-4, f"{what}: repeated call differs"
    if check_bf16:
        yb = dl.gemv(xd, td, torch.bfloat16)
        torch.cuda.synchronize()
        _check_y(yb, y_ref, TOL_BF16, what + " bf16")
        # bf16 output is the fp32 result rounded to nearest even.  The slices
        # are added in whatever order they arrive, so the fp32 value of this
        # call may differ from y in its last bits, by at most the fp32
        # rounding of its sums.  At the launch shapes of these cases (slices
        # of at least 64 channels, so at most 64 channels per worker and 64
        # slices) no chain of additions is 128 long, and each addition is off
        # by at most 2^-24 of the output's term magnitude
        # M_j = sum_i |x_i| (|s_j| (code_ij + phi_i) + |z_j|) over loaded
        # channels, so two calls differ by at most 2^-16 M_j.  Every output
        # must lie between the RNE roundings of y - delta and y + delta, with
        # delta that bound plus the spread seen between the two fp32 calls.
        # M_j is often hundreds of times |y_j| (the phi and z terms cancel), so
        # that bound is loose; the outputs whose rounding actually flips are
        # few, and at most 1% may differ from the RNE rounding of y itself.
        # (With one slice the result is deterministic and the check is exact:
        # test_gemv_bf16_is_rne_with_one_slice; the exact-integer tests pin
        # it at every slice count.)
        got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
        gotf = S.bf16_bits_to_f32(got).astype(np.float64)
        x_seen = x_f32 if x_dtype == "f32" else S.bf16_bits_to_f32(S.f32_to_bf16_bits(np.asarray(x_f32, np.float32)))
        mag = C.gemv(np.abs(np.asarray(x_seen, np.float32)), theta, dl.q_np, np.abs(dl.s_np), np.abs(dl.z_np),
                     dl.b_max)
        delta = 4.0 * np.abs(y2 - y) + 2.0 ** -16 * mag
        lo = S.bf16_bits_to_f32(O.round_to_bf16((y - delta).astype(np.float32))).astype(np.float64)
        hi = S.bf16_bits_to_f32(O.round_to_bf16((y + delta).astype(np.float32))).astype(np.float64)
        ok = (gotf >= lo) & (gotf <= hi)
        assert np.all(ok), f"{what}: bf16 output is not RNE of the fp32 output at {np.flatnonzero(~ok)[:8]}"
        rne = O.round_to_bf16(y.astype(np.float32))
        assert np.mean(got == rne) >= 0.99, f"{what}: bf16 output is not RNE of the fp32 output"
    return y


# ------------------------------------------------------------- packing ------

@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
@pytest.mark.parametrize("d_in,d_out", [(1, 1), (5, 1), (3, 65), (70, 130), (257, 1000), (1024, 1024),
                                        (65, 64)])
def test_pack_bit_exact(dev, b_max, d_in, d_out):
    say(f"pack b_max={b_max} d_in={d_in} d_out={d_out}")
    rng = np.random.default_rng(d_in * 7919 + d_out * 31 + b_max)
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)    # high bits must be masked
    dl = DeviceLinear(q, np.ones(d_out, np.float16), np.zeros(d_out, np.float16), b_max, dev)
    assert np.array_equal(dl.planes_np(), C.pack_planes(q, b_max))


# ------------------------------------------------------ bit assignment ------

def _assign_check(x_f32, x_dtype, theta, b_max, dev, what):
    import torch
    import input_adaptive_bit_amd as G
    say(f"assign {what}")
    x_f32 = np.asarray(x_f32, np.float32)
    L = G.grinqh_layout_init(x_f32.size, 64, b_max)
    bits, idx, n = G.assign_bits(L, to_dev_x(x_f32, x_dtype, dev), _theta_dev(theta, dev))
    torch.cuda.synchronize()
    x_seen = x_f32 if x_dtype == "f32" else S.bf16_bits_to_f32(S.f32_to_bf16_bits(x_f32))
    ref = O.assign_bits(x_seen, theta, b_max)
    got = bits.cpu().numpy()
    assert np.array_equal(got, ref)
    act = O.active_channels(ref)
    n_got = int(n.cpu().item())
    assert n_got == act.size
    assert np.array_equal(idx.cpu().numpy()[:n_got], act)


def test_assign_small_case(dev):
    L = S.make_linear(S.small_case(), with_codes=False)
    _assign_check(L.x, "f32", L.theta, 8, dev, "small case fp32")


@pytest.mark.parametrize("d_in", [1, 63, 64, 1025, 3000, 14336])
@pytest.mark.parametrize("b_max", [2, 4, 8])
def test_assign_bf16_ragged(dev, d_in, b_max):
    rng = np.random.default_rng(d_in + b_max)
    x = rng.standard_t(3, d_in).astype(np.float32)
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
    _assign_check(x, "bf16", theta, b_max, dev, f"bf16 d_in={d_in} b_max={b_max}")


def test_assign_special_values(dev, golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "assign_bits_ties.json")))
    x = np.array([float(v) for v in g["x"]], np.float32)
    _assign_check(x, "f32", np.array(g["theta"], np.float32), 8, dev, "golden ties fp32")
    _assign_check(x, "bf16", np.array(g["theta"], np.float32), 8, dev, "golden ties bf16")
    z = np.zeros(100, np.float32)
    _assign_check(z, "f32", np.zeros(4, np.float32), 8, dev, "dense zeros")
    _assign_check(np.ones(100, np.float32), "f32", np.full(4, np.inf, np.float32), 8, dev, "all skipped")


# ------------------------------------------------------------- codes --------

@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_debug_codes_bit_exact(dev, b_max):
    import torch
    import input_adaptive_bit_amd as G
    say(f"debug codes b_max={b_max}")
    rng = np.random.default_rng(50 + b_max)
    d_in, d_out = 300, 1000
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    x = rng.standard_normal(d_in).astype(np.float32)
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.15, 0.85, b_max // 2))).astype(np.float32)
    dl = DeviceLinear(q, np.ones(d_out, np.float16), np.zeros(d_out, np.float16), b_max, dev)
    bits, _, _ = G.assign_bits(dl.L, to_dev_x(x, "f32", dev), _theta_dev(theta, dev))
    codes = G.debug_codes(dl.L, bits, dl.planes)
    torch.cuda.synchronize()
    ref_bits = O.assign_bits(x, theta, b_max)
    ref = O.truncated_codes(q, ref_bits, b_max)
    assert np.array_equal(codes.cpu().numpy().astype(np.int64), ref)


# -------------------------------------------------------------- GEMV --------

def test_gemv_small_case(dev):
    L = S.make_linear(S.small_case())
    say("gemv small case 1024x1024 fp32 x")
    dl = DeviceLinear(L.q, L.s, L.z, 8, dev)
    y_ref = O.gemv(L.x, L.theta, L.q, L.s, L.z, 8, exact=True)
    _run_and_check(dl, L.x, "f32", L.theta, y_ref, "small case", dev)


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_gemv_bf16_is_rne_with_one_slice(dev, forced_shape, b_max, x_dtype):
    """With one slice per tile (d_in <= 256 at the longest slice) each tile's
    sums are one fixed-order LDS reduction and one add to zero, so the fp32
    result is the same on every call and the bf16 output must be its RNE
    rounding at every output."""
    import torch
    forced_shape(0, 256)
    rng = np.random.default_rng(900 + b_max)
    for d_in, d_out in [(1, 65), (100, 1000), (256, 4100)]:
        say(f"bf16 one slice b_max={b_max} {d_in}->{d_out} x={x_dtype}")
        q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
        s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
        z = rng.normal(0, 0.01, d_out).astype(np.float16)
        x = rng.standard_t(3, d_in).astype(np.float32)
        if x_dtype == "bf16":
            x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
        theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
        dl = DeviceLinear(q, s, z, b_max, dev)
        xd, td = to_dev_x(x, x_dtype, dev), _theta_dev(theta, dev)
        y1 = dl.gemv(xd, td, torch.float32)
        y2 = dl.gemv(xd, td, torch.float32)
        yb = dl.gemv(xd, td, torch.bfloat16)
        torch.cuda.synchronize()
        y1n = y1.cpu().numpy()
        _check_y(y1, C.gemv(x, theta, q, s, z, b_max), TOL_F32, "one slice fp32")
        assert np.array_equal(y1n.view(np.uint32), y2.cpu().numpy().view(np.uint32)), "one slice: calls differ"
        got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, O.round_to_bf16(y1n)), "one slice: bf16 output is not RNE of the fp32 output"


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
@pytest.mark.parametrize("d_in,d_out", [(1, 1), (1, 65), (3, 1), (17, 100), (300, 1500), (1000, 64),
                                        (2049, 3000)])
@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
def test_gemv_ragged_shapes(dev, b_max, d_in, d_out, x_dtype):
    say(f"gemv ragged b_max={b_max} {d_in}->{d_out} x={x_dtype}")
    rng = np.random.default_rng(d_in * 131 + d_out * 7 + b_max)
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = rng.standard_t(3, d_in).astype(np.float32)
    if x_dtype == "bf16":
        x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
    dl = DeviceLinear(q, s, z, b_max, dev)
    y_ref = C.gemv(x, theta, q, s, z, b_max)
    _run_and_check(dl, x, x_dtype, theta, y_ref, f"{d_in}->{d_out} b{b_max}", dev)


@pytest.mark.parametrize("d_in,d_out", [(66000, 100), (3000, 5000)])
def test_gemv_one_channel_slices(dev, forced_shape, d_in, d_out):
    """Slices of one channel: every input channel is its own workgroup.  At
    66000 channels the item count times the slice count passes 2^32, so the
    kernel takes a workgroup's tile by integer division instead of the
    host's multiply-high reciprocal; at 3000 x 5000 (20 tiles) it uses the
    reciprocal over 60000 items."""
    import torch
    forced_shape(8, 1)
    rng = np.random.default_rng(d_in + d_out)
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, 4))).astype(np.float32)
    say(f"one-channel slices {d_in}->{d_out}")
    dl = DeviceLinear(q, s, z, 8, dev)
    y = dl.gemv(to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), torch.float32)
    torch.cuda.synchronize()
    _check_y(y, C.gemv(x, theta, q, s, z, 8), TOL_F32, f"one-channel slices {d_in}->{d_out}")


@pytest.mark.parametrize("lane_groups", [1, 2, 4, 8])
@pytest.mark.parametrize("chunk", [7, 64, 256])
@pytest.mark.parametrize("b_max", [8, 4])
def test_gemv_forced_launch_shapes(dev, forced_shape, lane_groups, chunk, b_max):
    """Every tile width (1, 2, 4 or 8 lane groups per wave) with a short, a
    mid and the longest slice length, forced through the library's test
    override (grinqh_debug_force_launch), on shapes with several tiles and slices and ragged tails and on
    a one-channel layout narrower than one tile: single calls and a group call
    against the oracle."""
    import torch
    import input_adaptive_bit_amd as G
    forced_shape(lane_groups, chunk)
    rng = np.random.default_rng(lane_groups * 1000 + chunk + b_max)
    members, ops, refs = [], [], []
    for d_in, d_out in [(1500, 2500), (513, 4100), (40, 70), (1, 65)]:
        say(f"forced G={lane_groups} chunk={chunk} b_max={b_max} {d_in}->{d_out}")
        q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
        s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
        z = rng.normal(0, 0.01, d_out).astype(np.float16)
        x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
        theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
        dl = DeviceLinear(q, s, z, b_max, dev)
        y_ref = C.gemv(x, theta, q, s, z, b_max)
        _run_and_check(dl, x, "bf16", theta, y_ref, f"G{lane_groups} c{chunk} {d_in}->{d_out}", dev,
                       check_bf16=False)
        members.append(dl)
        ops.append((to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), dl.planes, dl.s, dl.z,
                    torch.empty(d_out, dtype=torch.float32, device=dev)))
        refs.append(y_ref)
    layouts = [m.L for m in members]
    ws = G.new_group_workspace(layouts, dev)
    G.grinqh_gemv_group(layouts, ops, ws)
    torch.cuda.synchronize()
    for k, (o, ref) in enumerate(zip(ops, refs)):
        got = o[5].cpu().numpy()
        err = O.max_rel_error(got, ref)
        assert err <= TOL_F32, (k, err, _mismatch(got, ref))


def test_gemv_dense_and_all_skipped(dev):
    import torch
    rng = np.random.default_rng(5)
    d_in, d_out = 777, 2000
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = rng.standard_normal(d_in).astype(np.float32)
    dl = DeviceLinear(q, s, z, 8, dev)
    say("gemv dense thresholds")
    th0 = np.zeros(4, np.float32)
    _run_and_check(dl, x, "f32", th0, C.gemv(x, th0, q, s, z, 8), "dense", dev)
    say("gemv all skipped")
    for th in (np.full(4, np.inf, np.float32), np.full(4, 1e30, np.float32)):
        y = dl.gemv(to_dev_x(x, "f32", dev), _theta_dev(th, dev), torch.float32)
        torch.cuda.synchronize()
        assert np.all(y.cpu().numpy() == 0.0)


def test_gemv_single_active_channel(dev):
    rng = np.random.default_rng(6)
    d_in, d_out = 500, 1100
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = np.full(d_in, 0.01, np.float32)
    x[321] = -3.0
    theta = np.array([1.0, 2.0, 2.5, 9.0], np.float32)
    dl = DeviceLinear(q, s, z, 8, dev)
    say("gemv single active channel")
    _run_and_check(dl, x, "f32", theta, C.gemv(x, theta, q, s, z, 8), "single channel", dev)


def test_gemv_nan_and_inf(dev):
    import torch
    rng = np.random.default_rng(8)
    d_in, d_out = 256, 256
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = rng.standard_normal(d_in).astype(np.float32)
    theta = np.array([0.2, 0.5, 1.0, 2.0], np.float32)
    dl = DeviceLinear(q, s, z, 8, dev)
    xn = x.copy()
    xn[7] = np.nan
    say("gemv NaN activation")
    _run_and_check(dl, xn, "f32", theta, C.gemv(xn, theta, q, s, z, 8), "nan channel skipped", dev)
    xi = x.copy()
    xi[9] = np.inf
    y = dl.gemv(to_dev_x(xi, "f32", dev), _theta_dev(theta, dev), torch.float32)
    torch.cuda.synchronize()
    assert not np.all(np.isfinite(y.cpu().numpy()))


def test_gemv_bruteforce_8x8(dev):
    """8 channels x 8 outputs (padded to 64), b_max 8: a seeded 1000-pattern
    subset of the 5^8 level patterns, the 5 uniform patterns and exact ties."""
    import torch
    rng = np.random.default_rng(88)
    q = rng.integers(0, 256, size=(8, 8), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, 8).astype(np.float16)
    z = rng.normal(0, 0.01, 8).astype(np.float16)
    theta = np.array([0.5, 1.0, 2.0, 4.0], np.float32)
    mid = np.array([0.25, 0.75, 1.5, 3.0, 6.0], np.float32)
    pats = [np.array(p) for p in rng.integers(0, 5, size=(1000, 8))]
    pats += [np.full(8, L) for L in range(5)]
    dl = DeviceLinear(q, s, z, 8, dev)
    td = _theta_dev(theta, dev)
    say("gemv brute force 8x8")
    xs = []
    for p in pats:
        sign = np.where(rng.random(8) < 0.5, -1.0, 1.0).astype(np.float32)
        xs.append(sign * mid[p])
    for k in range(20):                             # exact ties |x| = theta_k
        xs.append(rng.choice(np.concatenate([theta, -theta, [0.0]]), 8).astype(np.float32))
    ys = [dl.gemv(to_dev_x(xv, "f32", dev), td, torch.float32) for xv in xs]
    torch.cuda.synchronize()
    worst = 0.0
    for xv, yd in zip(xs, ys):
        ref = O.gemv(xv, theta, q, s, z, 8, exact=True)
        err = O.max_rel_error(yd.cpu().numpy(), ref) if np.any(ref != 0) else float(np.max(np.abs(yd.cpu().numpy())))
        worst = max(worst, err)
    say(f"  worst rel err {worst:.3e}")
    assert worst <= TOL_F32


def test_gemv_power_of_two_scaling_general_inputs(dev):
    """Heavy-tailed x: scaling x and theta by 2^m keeps b and the codes and
    scales y by 2^m up to the fp32 rounding of the slice sums, whose order
    between calls is not fixed (exact scaling, with exact sums, is checked in
    test_gpu_reduction)."""
    import torch
    rng = np.random.default_rng(9)
    d_in, d_out = 1500, 2100
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
    theta = np.sort(np.quantile(np.abs(x), [0.2, 0.5, 0.8, 0.95])).astype(np.float32)
    dl = DeviceLinear(q, s, z, 8, dev)
    say("gemv power-of-two scaling")
    y0 = dl.gemv(to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), torch.float32)
    for m in (-4, 3):
        ym = dl.gemv(to_dev_x(np.ldexp(x, m).astype(np.float32), "bf16", dev),
                     _theta_dev(np.ldexp(theta, m).astype(np.float32), dev), torch.float32)
        torch.cuda.synchronize()
        # same bits, same codes; y scales by 2^m up to the order of the slice sums
        assert O.max_rel_error((ym / (2.0 ** m)).cpu().numpy(), y0.cpu().numpy()) <= 5e-4


# ------------------------------------------------- full-size workloads ------

def _full_linear_check(spec, dev, sample=None):
    import torch
    L = S.make_linear(spec)
    say(f"full {spec.d_in}->{spec.d_out} b_max={spec.b_max} key={spec.key} q={spec.quantiles}")
    dl = DeviceLinear(L.q, L.s, L.z, spec.b_max, dev)
    xd = to_dev_x(L.x, spec.x_dtype, dev)
    y = dl.gemv(xd, _theta_dev(L.theta, dev), torch.float32)
    yb = dl.gemv(xd, _theta_dev(L.theta, dev), torch.bfloat16)
    torch.cuda.synchronize()
    cols = np.arange(spec.d_out) if sample is None else sample
    ref = C.gemv(L.x, L.theta, L.q[cols], L.s[cols], L.z[cols], spec.b_max)
    _check_y(y[torch.from_numpy(cols).to(dev)], ref, TOL_F32, "fp32")
    _check_y(yb[torch.from_numpy(cols).to(dev)], ref, TOL_BF16, "bf16")
    bits = O.assign_bits(L.x, L.theta, spec.b_max)
    say(f"  eff bits {O.eff_bits(bits):.3f}")
    del dl
    torch.cuda.empty_cache()


@pytest.mark.parametrize("eff", [2, 3, 4, 8])
def test_full_llama8b_linears(dev, eff):
    for spec in S.llama8b_linears(eff):
        _full_linear_check(spec, dev)


@pytest.mark.parametrize("eff", [2, 3, 6])
def test_full_llama8b_linears_b6(dev, eff):
    for spec in S.llama8b_linears_b6(eff):
        _full_linear_check(spec, dev)


@pytest.mark.parametrize("eff", [1.5, 2, 3, 4])
def test_full_llama8b_linears_b4(dev, eff):
    for spec in S.llama8b_linears_b4(eff):
        _full_linear_check(spec, dev)


@pytest.mark.parametrize("eff", [2, 3])
def test_full_llama70b_linears(dev, eff):
    rng = np.random.default_rng(70)
    for spec in S.llama70b_linears(eff):
        cols = np.unique(np.concatenate([[0, spec.d_out - 1], rng.integers(0, spec.d_out, 1024)]))
        _full_linear_check(spec, dev, sample=cols)


@pytest.mark.parametrize("eff,n_layers", [(3, 32), (2, 2), (4, 2), (6, 2), (8, 2)])
def test_full_decode_step_sampled(dev, eff, n_layers):
    """Every projection of the 32-layer 8B decode step as the benchmark
    launches it (fused q|k|v 4096->6144, o, fused gate|up 4096->28672, down;
    codes drawn on the device from a seeded generator), 64 sampled outputs of
    each checked against the oracle on the same code rows."""
    import torch
    specs = S.llama8b_decode_step(eff, n_layers)
    say(f"decode step eff={eff} layers={n_layers} linears={len(specs)}")
    worst = 0.0
    for spec in specs:
        g = torch.Generator(device=dev)
        g.manual_seed(S.torch_seed(spec.key, 0))
        q_dev = torch.randint(0, 256, (spec.d_out, spec.d_in), generator=g, dtype=torch.uint8, device=dev)
        Lin = S.make_linear(spec, with_codes=False)
        dl = DeviceLinear(None, Lin.s, Lin.z, 8, dev, q_dev=q_dev)
        y = dl.gemv(to_dev_x(Lin.x, "bf16", dev), _theta_dev(Lin.theta, dev), torch.float32)
        rng = np.random.default_rng(spec.key[2] * 10 + spec.key[3])
        cols = np.unique(np.concatenate([[0, spec.d_out - 1], rng.integers(0, spec.d_out, 64)]))
        cols_t = torch.from_numpy(cols).to(dev)
        q_rows = q_dev.index_select(0, cols_t).cpu().numpy()
        ref = C.gemv(Lin.x, Lin.theta, q_rows, Lin.s[cols], Lin.z[cols], 8)
        err = O.max_rel_error(y[cols_t].cpu().numpy(), ref)
        worst = max(worst, err)
        assert err <= TOL_F32, (spec, err)
        del dl, q_dev
    say(f"  worst rel err {worst:.3e}")


def test_gemv_graph_replays_match_eager(dev):
    """The GEMV captured in a HIP graph: every replay, with eager work and
    synchronisations in between, matches the eager call (the kernels use no
    memset; the workspace clears itself)."""
    import torch
    rng = np.random.default_rng(10)
    d_in, d_out = 4096, 4096
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
    theta = np.sort(np.quantile(np.abs(x), [0.2, 0.52, 0.82, 0.96])).astype(np.float32)
    dl = DeviceLinear(q, s, z, 8, dev)
    xd = to_dev_x(x, "bf16", dev)
    td = _theta_dev(theta, dev)
    say("gemv graph replays")
    eager = dl.gemv(xd, td, torch.float32).clone()
    y_ref = C.gemv(x, theta, q, s, z, 8)
    import input_adaptive_bit_amd as G
    y = torch.empty(d_out, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        G.grinqh_gemv(dl.L, xd, td, dl.planes, dl.s, dl.z, y, dl.ws)
    for rep in range(5):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert O.max_rel_error(got, eager.cpu().numpy()) <= 5e-4, rep
        assert O.max_rel_error(got, y_ref) <= TOL_F32, rep
        _ = dl.gemv(xd, td, torch.float32)      # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("d_in,d_out", [(4096, 14336), (14336, 4096), (4096, 4096)])
def test_gemv_exact_integer_sums_many_calls(dev, d_in, d_out):
    """Small-integer activations, s = 1, z = 1: every partial sum is a multiple
    of 1/2 below 2^23, so fp32 accumulation is exact in any order and y must
    equal the oracle exactly on every one of 20 back-to-back calls (a lost or
    stale cross-workgroup update would show as a mismatch)."""
    import torch
    rng = np.random.default_rng(d_in + d_out)
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = np.ones(d_out, np.float16)
    z = np.ones(d_out, np.float16)
    theta = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
    dl = DeviceLinear(q, s, z, 8, dev)
    td = _theta_dev(theta, dev)
    say(f"exact integer sums {d_in}->{d_out}")
    xs = [rng.choice(np.array([0.5, 1, 2, 3, 4, -1, -2, -3, -4, -0.5], np.float32), d_in) for _ in range(20)]
    outs = [dl.gemv(to_dev_x(x, "bf16", dev), td, torch.float32) for x in xs]
    torch.cuda.synchronize()
    for n, (x, y) in enumerate(zip(xs, outs)):
        ref = C.gemv(x, theta, q, s, z, 8)
        assert np.max(np.abs(ref)) < 2 ** 23
        got = y.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), (n, int(np.sum(got != ref)))


@pytest.mark.parametrize("d_in,d_out,b_max", [(1 << 20, 64, 8), (16, 1 << 20, 4)])
def test_gemv_maximum_dimensions(dev, d_in, d_out, b_max):
    """The largest d_in and d_out the library accepts (2^20): thousands of
    slices accumulating into one tile, and thousands of tiles of one slice."""
    import torch
    say(f"gemv maximum dimensions {d_in}->{d_out} b_max={b_max}")
    g = torch.Generator(device=dev)
    g.manual_seed(d_in + d_out)
    q_d = torch.randint(0, 1 << b_max, (d_out, d_in), dtype=torch.uint8, device=dev, generator=g)
    rng = np.random.default_rng(d_in + d_out)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
    dl = DeviceLinear(None, s, z, b_max, dev, q_dev=q_d)
    y = dl.gemv(to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), torch.float32)
    torch.cuda.synchronize()
    ref = C.gemv(x, theta, q_d.cpu().numpy(), s, z, b_max)
    err = O.max_rel_error(y.cpu().numpy(), ref)
    say(f"  max rel err {err:.3e}")
    assert err <= TOL_F32, (err, _mismatch(y.cpu().numpy(), ref))


def test_gemv_group_of_eight(dev):
    """A group of the maximum size (8 members), ragged shapes, against the oracle."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(88)
    shapes = [(4096, 4096), (1, 1), (777, 1000), (64, 65), (3000, 130), (8, 4100), (14336, 256), (129, 64)]
    members, ops, refs = [], [], []
    say("group launch of 8 members")
    for di, do in shapes:
        q = rng.integers(0, 256, size=(do, di), dtype=np.uint8)
        s = rng.uniform(0.001, 0.01, do).astype(np.float16)
        z = rng.normal(0, 0.01, do).astype(np.float16)
        x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, di).astype(np.float32)))
        theta = np.sort(np.quantile(np.abs(x), (0.2, 0.5, 0.8, 0.95))).astype(np.float32)
        dl = DeviceLinear(q, s, z, 8, dev)
        members.append(dl)
        ops.append((to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), dl.planes, dl.s, dl.z,
                    torch.empty(do, dtype=torch.float32, device=dev)))
        refs.append(C.gemv(x, theta, q, s, z, 8))
    layouts = [m.L for m in members]
    ws = G.new_group_workspace(layouts, dev)
    for rep in range(2):
        G.grinqh_gemv_group(layouts, ops, ws)
        torch.cuda.synchronize()
        for k, (o, ref) in enumerate(zip(ops, refs)):
            got = o[5].cpu().numpy()
            err = O.max_rel_error(got, ref)
            assert err <= TOL_F32, (rep, k, err, _mismatch(got, ref))


@pytest.mark.parametrize("b_max", [6, 8])
def test_gemv_slices_with_only_full_channels(dev, b_max):
    """Slices whose loaded channels all take every plane go down their own
    path (only the top bucket streamed); the other slices of the same launch
    take the general one.  Small-integer activations with s = z = 1 make the
    sums exact, so y must equal the oracle exactly: for x whose first half
    holds only full or skipped channels (both paths in one launch), for x
    where every slice is full, and for zero thresholds (every channel full),
    on single calls and on a group launch of the three."""
    import torch
    import input_adaptive_bit_amd as G
    P = b_max // 2
    rng = np.random.default_rng(400 + b_max)
    d_in, d_out = 4096 + 77, 2000
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    s = np.ones(d_out, np.float16)
    z = np.ones(d_out, np.float16)
    theta = np.arange(1, P + 1, dtype=np.float32)
    full = np.array([0.0, P, -P, P + 1, -(P + 1)], np.float32)            # 0 bits or b_max
    mixed = np.array([0.5, 1, -1, 2, -2, 3, -3, 4, -4, 0], np.float32)
    x_half = np.concatenate([rng.choice(full, d_in // 2), rng.choice(mixed, d_in - d_in // 2)])
    x_full = rng.choice(full, d_in)
    x_small = rng.choice(mixed, d_in)
    cases = [(x_half, theta), (x_full, theta), (x_small, np.zeros(P, np.float32))]
    dl = DeviceLinear(q, s, z, b_max, dev)
    say(f"gemv slices with only full channels b_max={b_max}")
    refs = [C.gemv(x, th, q, s, z, b_max) for x, th in cases]
    for ref in refs:
        assert np.max(np.abs(ref)) < 2 ** 23
    devs = [(to_dev_x(x, "bf16", dev), _theta_dev(th, dev)) for x, th in cases]
    for rep in range(3):
        outs = [dl.gemv(xd, td, torch.float32) for xd, td in devs]
        torch.cuda.synchronize()
        for k, (y, ref) in enumerate(zip(outs, refs)):
            got = y.cpu().numpy().astype(np.float64)
            assert np.array_equal(got, ref), (rep, k, int(np.sum(got != ref)))
    layouts = [dl.L] * 3
    ys = [torch.empty(d_out, dtype=torch.float32, device=dev) for _ in cases]
    ops = [(xd, td, dl.planes, dl.s, dl.z, y) for (xd, td), y in zip(devs, ys)]
    ws = G.new_group_workspace(layouts, dev)
    for rep in range(2):
        for y in ys:
            y.fill_(float("nan"))
        G.grinqh_gemv_group(layouts, ops, ws)
        torch.cuda.synchronize()
        for k, (y, ref) in enumerate(zip(ys, refs)):
            got = y.cpu().numpy().astype(np.float64)
            assert np.array_equal(got, ref), ("group", rep, k, int(np.sum(got != ref)))


@pytest.mark.parametrize("lane_groups", [1, 2, 4, 8])
def test_gemv_full_channel_slices_at_every_tile_width(dev, forced_shape, lane_groups):
    """The path of slices whose loaded channels all take every plane, at each
    tile width and with short slices (96 channels, so the top bucket needs
    several batches and a ragged last one): exact integer sums against the
    oracle at b_max 8 and 6, with half the slices on that path and half on the
    general one."""
    import torch
    d_in, d_out = 1000, 777
    forced_shape(lane_groups, 96)
    for b_max in (8, 6):
        P = b_max // 2
        rng = np.random.default_rng(500 + 10 * lane_groups + b_max)
        q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
        s = np.ones(d_out, np.float16)
        z = np.ones(d_out, np.float16)
        theta = np.arange(1, P + 1, dtype=np.float32)
        full = np.array([0.0, P, -P, P + 1, -(P + 1)], np.float32)
        mixed = np.array([0.5, 1, -1, 2, -2, 3, -3, 4, -4, 0], np.float32)
        x = np.concatenate([rng.choice(full, d_in // 2), rng.choice(mixed, d_in - d_in // 2)])
        dl = DeviceLinear(q, s, z, b_max, dev)
        say(f"full-channel slices G={lane_groups} b_max={b_max}")
        ref = C.gemv(x, theta, q, s, z, b_max)
        assert np.max(np.abs(ref)) < 2 ** 23
        y = dl.gemv(to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), torch.float32)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), (b_max, int(np.sum(got != ref)))


def test_gemv_early_batch_forms_at_their_thresholds(dev, forced_shape):
    """Slices whose four- and three-plane buckets sit just below and at the
    sizes where the early batches switch from skipping empty slots to the
    exact-wait form (32 and 48 entries at 4 lane groups, 256-channel slices):
    exact integer sums against the oracle, with both forms in one launch."""
    import torch
    forced_shape(4, 256)
    b_max, P = 8, 4
    rng = np.random.default_rng(777)
    # per 256-channel slice: (four-plane, three-plane) channel counts; the rest
    # of the slice is split between one- and two-plane channels and skipped ones
    plan = [(31, 47), (32, 47), (31, 48), (32, 48), (0, 0), (5, 60), (40, 10), (16, 24)]
    theta = np.array([1.0, 2.0, 3.0, 4.0], np.float32)
    mags = {4: [4.0, 5.0], 3: [3.0], 2: [2.0], 1: [1.0, 0.5 + 1.0], 0: [0.0, 0.5]}
    x = []
    for n4, n3 in plan:
        rest = 256 - n4 - n3
        lv = [4] * n4 + [3] * n3 + list(rng.choice([0, 1, 2], rest))
        rng.shuffle(lv)
        for l in lv:
            m = rng.choice(mags[l])
            x.append(m if rng.random() < 0.5 else -m)
    x = np.array(x, np.float32)
    d_in, d_out = x.size, 1536
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    s = np.ones(d_out, np.float16)
    z = np.ones(d_out, np.float16)
    dl = DeviceLinear(q, s, z, b_max, dev)
    say("early batch forms at their thresholds")
    ref = C.gemv(x, theta, q, s, z, b_max)
    assert np.max(np.abs(ref)) < 2 ** 23
    bits = 2 * (theta[None, :] <= np.abs(x)[:, None]).sum(1)
    for k, (n4, n3) in enumerate(plan):
        seg = bits[k * 256:(k + 1) * 256]
        assert (seg == 8).sum() == n4 and (seg == 6).sum() == n3
    for rep in range(3):
        y = dl.gemv(to_dev_x(x, "bf16", dev), _theta_dev(theta, dev), torch.float32)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref), (rep, int(np.sum(got != ref)))
