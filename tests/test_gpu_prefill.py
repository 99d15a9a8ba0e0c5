"""GPU parity of the prefill-stage dense b_max GEMM (grinqh_prefill_gemm,
through the C ABI) against the fp64 CPU oracle.

Every output row is held to the decode tolerance (max relative error 2e-3,
denominator max(|y*|, 1e-2 * rms of the row)); integer cases whose sums stay
below 2^24 must be bit-exact (the products are exact and every partial sum
is an integer that fp32 holds).
"""

import numpy as np
import pytest

from oracle import grinqh_oracle as O
import synthetic as S
from tests.gpu_util import TOL_BF16, TOL_F32, DeviceLinear, require_gpu, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import input_adaptive_bit_amd as G
    G.load()
    return require_gpu()


def _x_dev(X32, dev):
    """bf16 X on the device and the exact fp32 values it holds."""
    import torch
    bits = S.f32_to_bf16_bits(np.ascontiguousarray(X32, np.float32))
    xd = torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    return xd, S.bf16_bits_to_f32(bits)


def _row_err(Y, R):
    return max(O.max_rel_error(Y[m], R[m]) for m in range(R.shape[0]))


def _inputs(rng, M, d_in, d_out, b_max):
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    X = rng.standard_t(3, size=(M, d_in)).astype(np.float32)
    X[:, ::53] *= 20.0                                   # outlier channels
    return q, s, z, X


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
@pytest.mark.parametrize("M,d_in,d_out", [(1, 8, 1), (5, 64, 130), (77, 200, 1000), (128, 1024, 1024),
                                          (300, 4104, 700), (129, 64, 257)])
def test_prefill_matches_oracle(dev, b_max, M, d_in, d_out):
    import torch
    import input_adaptive_bit_amd as G
    say(f"prefill b_max={b_max} M={M} {d_in}->{d_out}")
    rng = np.random.default_rng(M * 7 + d_in * 3 + d_out + b_max)
    q, s, z, X = _inputs(rng, M, d_in, d_out, b_max)
    dl = DeviceLinear(q, s, z, b_max, dev)
    xd, Xh = _x_dev(X, dev)
    y32 = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    yb = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.bfloat16)
    torch.cuda.synchronize()
    R = O.prefill_gemm(Xh, q, s, z, b_max)
    Y = y32.cpu().numpy().astype(np.float64)
    err = _row_err(Y, R)
    say(f"  fp32 max row rel err {err:.3e}")
    assert err <= TOL_F32
    Yb = yb.float().cpu().numpy().astype(np.float64)
    assert _row_err(Yb, R) <= TOL_BF16
    # bf16 output is the fp32 result rounded to nearest even (the two calls
    # run the same kernel on the same inputs, so their fp32 values agree)
    rne = O.round_to_bf16(Y.astype(np.float32))
    got = yb.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, rne)


def test_prefill_output_store_paths_agree(dev):
    """y leaves through LDS as 16-byte row segments when y is 16-byte aligned
    and d_out a multiple of 16 bytes' worth of outputs, else element by
    element; a y view 2 bytes into its buffer takes the second path, and both
    must give the same bits."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(41)
    M, d_in, d_out = 300, 520, 1024
    say(f"prefill store paths M={M} {d_in}->{d_out}")
    q, s, z, X = _inputs(rng, M, d_in, d_out, 8)
    dl = DeviceLinear(q, s, z, 8, dev)
    xd, Xh = _x_dev(X, dev)
    ws = torch.empty(max(G.grinqh_prefill_workspace_bytes(M), 256), dtype=torch.uint8, device=dev)
    R = O.prefill_gemm(Xh, q, s, z, 8)
    for dt, tol in ((torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)):
        y_vec = torch.empty((M, d_out), dtype=dt, device=dev)
        buf = torch.empty(M * d_out + 8, dtype=dt, device=dev)
        y_el = buf[1:1 + M * d_out].view(M, d_out)
        assert y_vec.data_ptr() % 16 == 0 and y_el.data_ptr() % 16 != 0
        G.grinqh_prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, y_vec, ws)
        G.grinqh_prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, y_el, ws)
        torch.cuda.synchronize()
        assert torch.equal(y_vec.view(torch.int16 if dt == torch.bfloat16 else torch.int32),
                           y_el.view(torch.int16 if dt == torch.bfloat16 else torch.int32))
        assert _row_err(y_vec.float().cpu().numpy().astype(np.float64), R) <= tol


def test_prefill_integer_case_is_exact(dev):
    """s = 1, z = 0 would leave Y = X (Q + 1/2)^T; with s = 2 and z = -1 every
    weight is the odd integer 2q and Y the integer X (2Q)^T, exactly."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(5)
    M, d_in, d_out = 200, 1032, 300
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    X = rng.integers(-4, 5, size=(M, d_in)).astype(np.float32)
    s = np.full(d_out, 2.0, np.float16)
    z = np.full(d_out, -1.0, np.float16)
    dl = DeviceLinear(q, s, z, 8, dev)
    xd, Xh = _x_dev(X, dev)
    y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    torch.cuda.synchronize()
    ref = (X.astype(np.int64) @ (2 * q.astype(np.int64)).T).astype(np.float64)
    assert np.max(np.abs(ref)) < 2 ** 23
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def test_prefill_degenerate_cases(dev):
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(6)
    M, d_in, d_out = 40, 136, 90
    q = rng.integers(0, 256, size=(d_out, d_in), dtype=np.uint8)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    X = rng.normal(size=(M, d_in)).astype(np.float32)
    # s = 0: every weight is z_j, so Y = z_j * (row sum of X)
    dl = DeviceLinear(q, np.zeros(d_out, np.float16), z, 8, dev)
    xd, Xh = _x_dev(X, dev)
    y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    # all-zero X gives exact zeros
    y0 = G.prefill_gemm(dl.L, torch.zeros_like(xd), dl.planes, dl.s, dl.z, torch.float32)
    torch.cuda.synchronize()
    R = O.prefill_gemm(Xh, q, np.zeros(d_out, np.float16), z, 8)
    assert _row_err(y.cpu().numpy().astype(np.float64), R) <= TOL_F32
    assert np.all(y0.cpu().numpy() == 0)


def test_prefill_single_token_matches_dense_decode(dev):
    """One token: the prefill row equals the decode GEMV with every channel
    loaded (thresholds 0) on the same planes, to fp32 summation order."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(7)
    for b_max in (4, 8):
        d_in, d_out = 4096, 4096
        q, s, z, X = _inputs(rng, 3, d_in, d_out, b_max)
        dl = DeviceLinear(q, s, z, b_max, dev)
        xd, Xh = _x_dev(X, dev)
        yp = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
        th = to_dev(np.zeros(b_max // 2, np.float32), dev)
        yd = [dl.gemv(xd[m].contiguous(), th, torch.float32) for m in range(3)]
        torch.cuda.synchronize()
        P = yp.cpu().numpy().astype(np.float64)
        for m in range(3):
            assert O.max_rel_error(P[m], yd[m].cpu().numpy().astype(np.float64)) <= 5e-4


def test_prefill_after_rtn(dev):
    """bf16 W -> RTN codes, scales and zero points -> pack -> prefill, against
    the oracle on the same codes."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(8)
    M, d_in, d_out = 96, 2048, 1536
    w32 = rng.normal(0, 0.02, size=(d_out, d_in)).astype(np.float32)
    wbits = S.f32_to_bf16_bits(w32)
    wd = torch.from_numpy(wbits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    q_d, s_d, z_d = G.quantize_rtn(wd, 8)
    q, s, z = q_d.cpu().numpy(), s_d.cpu().numpy(), z_d.cpu().numpy()
    dl = DeviceLinear(None, s, z, 8, dev, q_dev=q_d)
    X = rng.standard_t(3, size=(M, d_in)).astype(np.float32)
    xd, Xh = _x_dev(X, dev)
    y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    torch.cuda.synchronize()
    R = O.prefill_gemm(Xh, q, s, z, 8)
    err = _row_err(y.cpu().numpy().astype(np.float64), R)
    say(f"  rtn -> prefill: max row rel err {err:.3e}")
    assert err <= TOL_F32


@pytest.mark.parametrize("b_max", [8, 4])
def test_prefill_full_size_sampled(dev, b_max):
    """The benchmark's workload, 2048 tokens through a 4096 -> 16384 up
    projection, in the benchmark's launch: 16 sampled token rows (tile edges
    among them), every output, against the oracle."""
    import torch
    import input_adaptive_bit_amd as G
    say(f"prefill full size 2048 x 4096 -> 16384 b_max={b_max}")
    M, d_in, d_out = 2048, 4096, 16384
    g = torch.Generator(device=dev)
    g.manual_seed(b_max)
    q_d = torch.randint(0, 1 << b_max, (d_out, d_in), dtype=torch.uint8, device=dev, generator=g)
    rng = np.random.default_rng(9 + b_max)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    X = rng.standard_t(3, size=(M, d_in)).astype(np.float32)
    dl = DeviceLinear(None, s, z, b_max, dev, q_dev=q_d)
    xd, Xh = _x_dev(X, dev)
    y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 127, 128, M - 1], rng.choice(np.arange(129, M - 1), 12, replace=False)]))
    R = O.prefill_gemm(Xh[rows], q_d.cpu().numpy(), s, z, b_max)     # whole rows, every output
    Y = y[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    err = _row_err(Y, R)
    say(f"  sampled rows: max rel err {err:.3e}")
    assert err <= TOL_BF16


@pytest.mark.parametrize("tile", [(128, 128), (256, 256), (256, 128)])
@pytest.mark.parametrize("b_max", [2, 8])
def test_prefill_forced_tiles(dev, tile, b_max):
    """Every tile shape (128 x 128, 256 x 256 and 256 x 128 tokens x outputs),
    forced through the library's test override (grinqh_debug_force_launch), on shapes with ragged token, channel and
    output tails; 300 x 136 -> 2048 has a multiple of 8 tile columns at every
    tile width (the XCD-grouped tile order) and several tile rows."""
    import torch
    import input_adaptive_bit_amd as G
    G.force_launch_shape(0, 0, tile)
    try:
        _forced_tile_cases(dev, tile, b_max)
    finally:
        G.force_launch_shape(0, 0, 0)


def _forced_tile_cases(dev, tile, b_max):
    import torch
    import input_adaptive_bit_amd as G
    for M, d_in, d_out in [(300, 4104, 700), (5, 64, 130), (257, 136, 513), (512, 512, 512), (300, 136, 2048)]:
        say(f"prefill forced tile {tile} b_max={b_max} M={M} {d_in}->{d_out}")
        rng = np.random.default_rng(tile[0] + tile[1] // 128 + b_max + M + d_in + d_out)
        q, s, z, X = _inputs(rng, M, d_in, d_out, b_max)
        dl = DeviceLinear(q, s, z, b_max, dev)
        xd, Xh = _x_dev(X, dev)
        y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
        yb = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.bfloat16)
        torch.cuda.synchronize()
        R = O.prefill_gemm(Xh, q, s, z, b_max)
        err = _row_err(y.cpu().numpy().astype(np.float64), R)
        assert err <= TOL_F32, (M, d_in, d_out, err)
        assert _row_err(yb.float().cpu().numpy().astype(np.float64), R) <= TOL_BF16, (M, d_in, d_out)


def test_prefill_maximum_token_count(dev):
    """2^20 tokens (the largest M the library accepts) through a narrow layer;
    sampled rows, the first and last among them, against the oracle."""
    import torch
    import input_adaptive_bit_amd as G
    M, d_in, d_out = 1 << 20, 8, 64
    say(f"prefill maximum token count M={M} {d_in}->{d_out}")
    rng = np.random.default_rng(20)
    q, s, z, X = _inputs(rng, M, d_in, d_out, 8)
    dl = DeviceLinear(q, s, z, 8, dev)
    xd, Xh = _x_dev(X, dev)
    y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    torch.cuda.synchronize()
    rows = np.sort(np.concatenate([[0, 255, 256, M - 1], rng.choice(M, 60, replace=False)]))
    R = O.prefill_gemm(Xh[rows], q, s, z, 8)
    Y = y[torch.from_numpy(rows).to(dev)].cpu().numpy().astype(np.float64)
    assert _row_err(Y, R) <= TOL_F32


def test_prefill_graph_replays_match_eager(dev):
    """The prefill call captured in a HIP graph: every replay, with eager work
    and synchronisations in between, equals the eager call bit for bit (no
    atomics: the summation order is fixed) and the oracle to tolerance."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(30)
    M, d_in, d_out = 600, 1024, 1500
    q, s, z, X = _inputs(rng, M, d_in, d_out, 8)
    dl = DeviceLinear(q, s, z, 8, dev)
    xd, Xh = _x_dev(X, dev)
    say("prefill graph replays")
    eager = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    R = O.prefill_gemm(Xh, q, s, z, 8)
    y = torch.empty((M, d_out), dtype=torch.float32, device=dev)
    ws = torch.empty(G.grinqh_prefill_workspace_bytes(M), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        G.grinqh_prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, y, ws)
    ref = eager.cpu().numpy()
    for rep in range(5):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got = y.cpu().numpy()
        assert np.array_equal(got, ref), rep
        assert _row_err(got.astype(np.float64), R) <= TOL_F32, rep
        _ = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)   # eager work between replays
        torch.cuda.synchronize()


def test_prefill_nan_and_inf_rows(dev):
    """A token row holding NaN or Inf gives non-finite outputs, as in the
    oracle; the other rows are unaffected."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(31)
    M, d_in, d_out = 40, 512, 300
    q, s, z, X = _inputs(rng, M, d_in, d_out, 8)
    X[3, 17] = np.nan
    X[7, 200] = np.inf
    X[11, 5] = -np.inf
    dl = DeviceLinear(q, s, z, 8, dev)
    xd, Xh = _x_dev(X, dev)
    y = G.prefill_gemm(dl.L, xd, dl.planes, dl.s, dl.z, torch.float32)
    torch.cuda.synchronize()
    Y = y.cpu().numpy().astype(np.float64)
    with np.errstate(invalid="ignore"):
        R = O.prefill_gemm(Xh, q, s, z, 8)
    bad = [3, 7, 11]
    assert np.all(~np.isfinite(Y[bad])) and np.all(~np.isfinite(R[bad]))
    good = [m for m in range(M) if m not in bad]
    assert np.all(np.isfinite(Y[good]))
    assert _row_err(Y[good], R[good]) <= TOL_F32
