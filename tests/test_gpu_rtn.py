"""GPU parity of the offline RTN front end (grinqh_quantize_rtn, through the C
ABI) against the CPU oracle: codes, scales and zero points bit-identical
(both sides take every rounding decision in fp32 with the stored fp16 scale
and zero point), and the codes feeding the decode GEMV end to end."""

import numpy as np
import pytest

from oracle import grinqh_oracle as O
from oracle import c_oracle as C
import synthetic as S
from tests.gpu_util import TOL_F32, DeviceLinear, require_gpu, say, to_dev, to_dev_x

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import input_adaptive_bit_amd as G
    G.load()
    return require_gpu()


def _bf16(w32):
    bits = S.f32_to_bf16_bits(np.asarray(w32, np.float32))
    return bits, S.bf16_bits_to_f32(bits)


def _run(w_bits, b_max, dev):
    import input_adaptive_bit_amd as G
    import torch
    wd = torch.from_numpy(w_bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    q, s, z = G.quantize_rtn(wd, b_max)
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy()


def _same_f16(a, b):
    a, b = np.asarray(a, np.float16), np.asarray(b, np.float16)
    both_nan = np.isnan(a) & np.isnan(b)
    return np.all(both_nan | (a.view(np.uint16) == b.view(np.uint16)))


def _check(w32, b_max, dev):
    bits, w = _bf16(w32)
    q, s, z = _run(bits, b_max, dev)
    qr, sr, zr = O.quantize_rtn(w, b_max)
    assert np.array_equal(q, qr), (b_max, np.argwhere(q != qr)[:5])
    assert _same_f16(s, sr) and _same_f16(z, zr)
    return q, s, z


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
@pytest.mark.parametrize("d_out,d_in", [(1, 1), (3, 7), (5, 8), (17, 1000), (9, 4096), (4, 14336), (64, 777)])
def test_rtn_matches_oracle(dev, b_max, d_out, d_in):
    say(f"rtn b_max={b_max} {d_out}x{d_in}")
    rng = np.random.default_rng(d_out * 31 + d_in + b_max)
    w = rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)
    w[:, ::97] *= 30.0                                    # outlier columns
    _check(w, b_max, dev)


def test_rtn_exact_grids_on_device(dev):
    """The oracle's exact-grid pins, run through the device: rows of known
    codes come back as those codes."""
    for k in (0, 3, 9):
        rng = np.random.default_rng(k)
        q_true = rng.integers(0, 256, size=(6, 300))
        w = (q_true * 2.0 ** -k).astype(np.float32)
        w[:, 0], w[:, 1] = 0.0, 256 * 2.0 ** -k
        q_true[:, 0], q_true[:, 1] = 0, 255
        q, s, z = _check(w, 8, dev)
        assert np.array_equal(q, q_true.astype(np.uint8)) and np.all(s == np.float16(2.0 ** -k))
    rng = np.random.default_rng(4)
    q_true = rng.integers(0, 16, size=(5, 200))
    w = ((q_true + 0.5) * 0.125).astype(np.float32)
    w[:, 0], w[:, 1] = 0.0, 2.0
    q_true[:, 0], q_true[:, 1] = 0, 15
    q, s, z = _check(w, 4, dev)
    assert np.array_equal(q, q_true.astype(np.uint8))


def test_rtn_special_rows_on_device(dev):
    w = np.array([[1.5] * 16,
                  [np.nan, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15],
                  [0, 1, np.inf, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14],
                  [np.nan] * 16,
                  [-0.0, 0.0] * 8,
                  [-np.inf, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 1e-30]], np.float32)
    for b_max in (2, 8):
        _check(w, b_max, dev)


def test_rtn_full_size_gate_projection(dev):
    say("rtn 14336x4096 (an 8B gate projection)")
    rng = np.random.default_rng(14336)
    w = rng.normal(0, 0.015, size=(14336, 4096)).astype(np.float32)
    w[rng.integers(0, 14336, 200), rng.integers(0, 4096, 200)] *= 50.0
    _check(w, 8, dev)


@pytest.mark.parametrize("b_max", [4, 8])
def test_rtn_then_decode_gemv(dev, b_max):
    """RTN codes, scales and zero points feed pack and the decode GEMV; the
    result matches the oracle GEMV on the same codes."""
    import torch
    d_out, d_in = 3000, 2049
    rng = np.random.default_rng(b_max)
    w32 = rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)
    bits, _ = _bf16(w32)
    wd = torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    import input_adaptive_bit_amd as G
    q_d, s_d, z_d = G.quantize_rtn(wd, b_max)
    q, s, z = q_d.cpu().numpy(), s_d.cpu().numpy(), z_d.cpu().numpy()
    dl = DeviceLinear(None, s, z, b_max, dev, q_dev=q_d)
    x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
    y = dl.gemv(to_dev_x(x, "bf16", dev), to_dev(theta, dev), torch.float32)
    ref = C.gemv(x, theta, q, s, z, b_max)
    err = O.max_rel_error(y.cpu().numpy(), ref)
    say(f"  rtn -> gemv b_max={b_max}: max rel err {err:.3e}")
    assert err <= TOL_F32


def test_rtn_graph_replays(dev):
    """RTN captured in a HIP graph: every replay, with eager work in between,
    gives the oracle's codes, scales and zero points bit for bit."""
    import input_adaptive_bit_amd as G
    import torch
    rng = np.random.default_rng(13)
    w = rng.normal(0, 0.02, size=(300, 2048)).astype(np.float32)
    bits, wf = _bf16(w)
    wd = torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    qr, sr, zr = O.quantize_rtn(wf, 8)
    q = torch.empty((300, 2048), dtype=torch.uint8, device=dev)
    s = torch.empty(300, dtype=torch.float16, device=dev)
    z = torch.empty(300, dtype=torch.float16, device=dev)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        G.grinqh_quantize_rtn(wd, 8, q, s, z)
    for rep in range(5):
        q.fill_(0)
        s.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(q.cpu().numpy(), qr), rep
        assert _same_f16(s.cpu().numpy(), sr) and _same_f16(z.cpu().numpy(), zr), rep
        _check(rng.normal(size=(7, 100)).astype(np.float32), 4, dev)             # eager work in between
