"""GPU tests of the GEMV's cross-workgroup reduction and epilogue (through
the C ABI): y_j = s_j * (A_j + C) + z_j * S, where every input-channel slice
adds its partial A_j + C and its partial S into the workspace and the last
workgroup to arrive at an output tile applies the epilogue.

* z*S dominant: tiny s and large z make y almost entirely z_j * S, so an
  epilogue that used a missing or stale S would be far off the oracle.  The
  shapes put live outputs in every wave of a tile at every tile width.
* Exact integer sums: small-integer activations with s = z = 1 make every
  partial sum a multiple of 1/4 far below 2^22, so fp32 accumulation is exact
  in any order; y must equal the fp64 oracle exactly on every call, at every
  b_max, for single calls and for grouped launches, and the bf16 output must
  be the exact result rounded to nearest even.
"""

import numpy as np
import pytest

from oracle import grinqh_oracle as O
from oracle import c_oracle as C
import synthetic as S
from tests.gpu_util import TOL_F32, DeviceLinear, require_gpu, say, to_dev, to_dev_x

pytestmark = pytest.mark.gpu

EXACT_X = np.array([0.5, 1, 2, 3, 4, -1, -2, -3, -4, -0.5], np.float32)


@pytest.fixture(scope="module")
def dev():
    import input_adaptive_bit_amd as G
    G.load()
    return require_gpu()


def _theta_dev(theta, dev):
    return to_dev(np.asarray(theta, np.float32), dev)


def _worst(got, ref, n=4):
    got = np.asarray(got, np.float64)
    d = np.abs(got - ref)
    idx = np.argsort(-d)[:n]
    return [(int(j), float(got[j]), float(ref[j])) for j in idx]


def _exact_theta(b_max):
    return np.array([1.0, 2.0, 3.0, 4.0][: b_max // 2], np.float32)


@pytest.mark.parametrize("lane_groups", [0, 1, 2, 4, 8])
@pytest.mark.parametrize("b_max", [8, 4])
def test_gemv_zs_dominant(dev, lane_groups, b_max):
    """Tiny s (1e-4) and z of order one: y is dominated by z_j * S.  Outputs
    live in every wave of a tile (d_out 65, 1000, 2100 at tile widths 64 to
    2048), each launch checked against the oracle; the default launch shape
    (0) and every forced tile width."""
    import torch
    import input_adaptive_bit_amd as G
    G.force_launch_shape(lane_groups, 0)
    try:
        rng = np.random.default_rng(500 + 10 * lane_groups + b_max)
        for d_in, d_out in [(1, 65), (300, 1000), (2049, 2100), (4096, 4096)]:
            say(f"z*S dominant G={lane_groups} b_max={b_max} {d_in}->{d_out}")
            q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
            s = np.full(d_out, 1e-4, np.float16)
            z = rng.uniform(0.5, 2.0, d_out).astype(np.float16) * np.where(rng.random(d_out) < 0.5, -1, 1)
            z = z.astype(np.float16)
            x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
            x[0] = 3.0                                # at least one loaded channel
            theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
            theta = np.minimum(theta, np.float32(3.0))
            dl = DeviceLinear(q, s, z, b_max, dev)
            ref = C.gemv(x, theta, q, s, z, b_max)
            xd, td = to_dev_x(x, "bf16", dev), _theta_dev(theta, dev)
            outs = [dl.gemv(xd, td, torch.float32) for _ in range(4)]
            torch.cuda.synchronize()
            for n, y in enumerate(outs):
                got = y.cpu().numpy()
                err = O.max_rel_error(got, ref)
                assert err <= TOL_F32, (n, err, _worst(got, ref))
    finally:
        G.force_launch_shape(0, 0)


def _exact_case(rng, d_in, d_out, b_max, n_x):
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    s = np.ones(d_out, np.float16)
    z = np.ones(d_out, np.float16)
    xs = [rng.choice(EXACT_X, d_in) for _ in range(n_x)]
    return q, s, z, xs


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_gemv_exact_integer_sums_every_bmax(dev, b_max):
    """Exact sums at every b_max on shapes with several tiles and slices and
    live outputs in every wave: 10 back-to-back calls per shape, each equal to
    the oracle exactly; the bf16 output equals the exact result rounded to
    nearest even, and scaling x and theta by 2^m scales y by exactly 2^m."""
    import torch
    rng = np.random.default_rng(900 + b_max)
    theta = _exact_theta(b_max)
    for d_in, d_out in [(4096, 4096), (14336, 1000), (300, 2100), (1, 65), (2049, 14336)]:
        say(f"exact sums b_max={b_max} {d_in}->{d_out}")
        q, s, z, xs = _exact_case(rng, d_in, d_out, b_max, 10)
        dl = DeviceLinear(q, s, z, b_max, dev)
        td = _theta_dev(theta, dev)
        outs = [dl.gemv(to_dev_x(x, "bf16", dev), td, torch.float32) for x in xs]
        torch.cuda.synchronize()
        refs = []
        for n, (x, y) in enumerate(zip(xs, outs)):
            ref = C.gemv(x, theta, q, s, z, b_max)
            assert np.max(np.abs(ref)) < 2 ** 21
            got = y.cpu().numpy().astype(np.float64)
            assert np.array_equal(got, ref), (n, int(np.sum(got != ref)), _worst(got, ref))
            refs.append(ref)
        yb = dl.gemv(to_dev_x(xs[0], "bf16", dev), td, torch.bfloat16)
        torch.cuda.synchronize()
        got_b = yb.view(torch.int16).cpu().numpy().view(np.uint16)
        want_b = O.round_to_bf16(refs[0].astype(np.float32))
        assert np.array_equal(got_b, want_b), int(np.sum(got_b != want_b))
        for m in (-3, 2):
            ym = dl.gemv(to_dev_x(np.ldexp(xs[0], m).astype(np.float32), "bf16", dev),
                         _theta_dev(np.ldexp(theta, m).astype(np.float32), dev), torch.float32)
            torch.cuda.synchronize()
            assert np.array_equal(ym.cpu().numpy().astype(np.float64), np.ldexp(refs[0], m)), m


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_gemv_group_exact_integer_sums(dev, b_max):
    """Grouped launches with exact sums: every member of every launch equals
    the oracle exactly (members of different shapes, including a one-channel
    65-output member and members with live outputs in every wave)."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(950 + b_max)
    theta = _exact_theta(b_max)
    shapes = [(4096, 4096), (4096, 1024), (1, 65), (300, 1000), (14336, 4096), (777, 2100)]
    members, qs, xss, outs = [], [], [], []
    say(f"group exact sums b_max={b_max}")
    for d_in, d_out in shapes:
        q, s, z, xs = _exact_case(rng, d_in, d_out, b_max, 5)
        members.append(DeviceLinear(q, s, z, b_max, dev))
        qs.append(q)
        xss.append(xs)
        outs.append(torch.empty(d_out, dtype=torch.float32, device=dev))
    layouts = [m.L for m in members]
    ws = G.new_group_workspace(layouts, dev)
    td = _theta_dev(theta, dev)
    for call in range(5):
        ops = [(to_dev_x(xss[k][call], "bf16", dev), td, m.planes, m.s, m.z, outs[k])
               for k, m in enumerate(members)]
        for o in outs:
            o.fill_(float("nan"))
        G.grinqh_gemv_group(layouts, ops, ws)
        torch.cuda.synchronize()
        for k, m in enumerate(members):
            ref = C.gemv(xss[k][call], theta, qs[k], np.ones(m.d_out, np.float16), np.ones(m.d_out, np.float16),
                         b_max)
            got = outs[k].cpu().numpy().astype(np.float64)
            assert np.array_equal(got, ref), (call, k, int(np.sum(got != ref)), _worst(got, ref))
