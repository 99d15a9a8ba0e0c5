"""GPU parity of the threshold calibration (grinqh_calibrate_thresholds, through
the C ABI) against the fp64 CPU oracle: the fp32 thresholds must be
bit-identical (the device finds the order statistics exactly and rounds the
same fp64 interpolation once)."""

import numpy as np
import pytest

from oracle import grinqh_oracle as O
import synthetic as S
from tests.gpu_util import require_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import input_adaptive_bit_amd as G
    G.load()
    return require_gpu()


def _device_x(x32, dtype, dev):
    import torch
    if dtype == "bf16":
        bits = S.f32_to_bf16_bits(np.asarray(x32, np.float32))
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16), S.bf16_bits_to_f32(bits)
    x = np.ascontiguousarray(np.asarray(x32, np.float32))
    return torch.from_numpy(x).to(dev), x


def _check(x32, levels, dtype, dev, ws=None):
    import input_adaptive_bit_amd as G
    import torch
    xd, xh = _device_x(x32, dtype, dev)
    got = G.calibrate_thresholds(xd, levels, ws)
    torch.cuda.synchronize()
    ref = O.calibrate_thresholds(xh, levels)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.int32), ref.view(np.int32)), (levels, g, ref)
    return g


LEVELS = [list(S.QUANTILES_B8[3]), [0.0, 1.0], [0.5], list(S.QUANTILES_B8[2]), [0.0, 0.3333, 0.6667, 1.0]]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n", [1, 2, 3, 7, 1000, 4096 * 3 + 7, 128 * 4096, 128 * 14336])
def test_calibration_matches_oracle(dev, dtype, n):
    say(f"calibration {dtype} n={n}")
    rng = np.random.default_rng(n + (7 if dtype == "f32" else 0))
    x = rng.standard_t(3, n).astype(np.float32) * np.float32(rng.uniform(0.1, 10))
    for lv in LEVELS:
        _check(x, lv, dtype, dev)


def test_calibration_ties_and_special_values(dev):
    import torch
    say("calibration ties and special values")
    rng = np.random.default_rng(3)
    ints = rng.integers(-6, 7, 20000).astype(np.float32)          # heavy ties, both signs
    for lv in LEVELS:
        _check(ints, lv, "f32", dev)
        _check(ints, lv, "bf16", dev)
    tiny = np.array([0.0, -0.0, 1e-45, -1e-42, 1e-40, 3.0, np.inf, -np.inf, np.nan, 2.5], np.float32)
    for lv in ([0.0, 0.1, 0.15, 0.3], [0.5, 0.7, 0.8, 0.89], [0.9, 1.0]):
        _check(tiny, lv, "f32", dev)
    # one value repeated
    _check(np.full(513, -0.75, np.float32), [0.0, 0.5, 1.0], "bf16", dev)


def test_calibration_on_the_harness_stream(dev):
    """The 128 calibration samples of a synthetic 8B linear: the device
    thresholds equal the oracle's and the harness's (numpy.quantile) to within
    one fp32 step."""
    say("calibration on the synthetic calibration stream")
    spec = S.llama8b_linears(3)[1]
    xs, _ = S.gen_x_stream(spec)
    calib = xs[:spec.n_calib]
    got = _check(calib, list(spec.quantiles), "bf16", dev)
    harness = S.calibrate_theta(S.bf16_bits_to_f32(S.f32_to_bf16_bits(calib)), spec.quantiles, 4)
    assert np.all(np.abs(got.view(np.int32).astype(np.int64) - harness.view(np.int32).astype(np.int64)) <= 1)


def test_calibration_workspace_reuse(dev):
    """Calls in a row on one workspace (any contents) give the same result."""
    import input_adaptive_bit_amd as G
    import torch
    ws = torch.full((G.grinqh_calibrate_workspace_bytes(),), 0xAB, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(11)
    for n in (50000, 37, 50000):
        x = rng.standard_t(3, n).astype(np.float32)
        _check(x, list(S.QUANTILES_B8[4]), "f32", dev, ws)


def test_calibration_graph_replays(dev):
    """Calibration captured in a HIP graph (its workspace is initialised by a
    kernel, no memset): every replay, with eager work in between, gives the
    oracle's thresholds bit for bit."""
    import input_adaptive_bit_amd as G
    import torch
    rng = np.random.default_rng(12)
    x = rng.standard_t(3, 128 * 1024).astype(np.float32)
    xd, xh = _device_x(x, "bf16", dev)
    lv = list(S.QUANTILES_B8[3])
    ref = O.calibrate_thresholds(xh, lv)
    ws = torch.empty(G.grinqh_calibrate_workspace_bytes(), dtype=torch.uint8, device=dev)
    th = torch.empty(len(lv), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        G.grinqh_calibrate_thresholds(xd, lv, th, ws)
    for rep in range(5):
        th.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(th.cpu().numpy().view(np.int32), ref.view(np.int32)), rep
        _check(rng.standard_t(3, 5000).astype(np.float32), [0.5], "f32", dev)     # eager work in between
