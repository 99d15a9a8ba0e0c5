"""GPU test of grinqh_gemv_noalloc (through the C ABI): the GEMV with the
library's static device workspace matches grinqh_gemv with a caller
workspace, on consecutive calls whose second input is smaller than the
first, and both match the fp64 oracle."""

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


def _case(rng, d_in, d_out, b_max, exact):
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    if exact:
        s = np.ones(d_out, np.float16)
        z = np.ones(d_out, np.float16)
        x = rng.choice(EXACT_X, d_in)
        theta = np.array([1.0, 2.0, 3.0, 4.0][: b_max // 2], np.float32)
    else:
        s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
        z = rng.normal(0, 0.01, d_out).astype(np.float16)
        x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(rng.standard_t(3, d_in).astype(np.float32)))
        theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
    return q, s, z, x, theta


@pytest.mark.parametrize("exact", [True, False])
@pytest.mark.parametrize("b_max", [8, 4])
def test_gemv_noalloc_matches_workspace_call(dev, b_max, exact):
    """Two calls in a row, the second on a smaller layer: each equals the
    workspace call exactly when the sums are exact, else agrees to fp32
    rounding of the slice-sum order; both within the oracle tolerance.  The
    bf16 output is checked on the second layer too."""
    import torch
    import input_adaptive_bit_amd as G
    rng = np.random.default_rng(4242 + b_max + 10 * exact)
    for d_in, d_out in [(14336, 4096), (300, 1000), (1, 65)]:
        say(f"noalloc b_max={b_max} exact={exact} {d_in}->{d_out}")
        q, s, z, x, theta = _case(rng, d_in, d_out, b_max, exact)
        dl = DeviceLinear(q, s, z, b_max, dev)
        xd, td = to_dev_x(x, "bf16", dev), to_dev(theta, dev)
        y_ws = torch.full((d_out,), float("nan"), dtype=torch.float32, device=dev)
        y_na = torch.full((d_out,), float("nan"), dtype=torch.float32, device=dev)
        G.grinqh_gemv(dl.L, xd, td, dl.planes, dl.s, dl.z, y_ws, dl.ws)
        G.grinqh_gemv_noalloc(dl.L, xd, td, dl.planes, dl.s, dl.z, y_na)
        yb_na = torch.empty(d_out, dtype=torch.bfloat16, device=dev)
        G.grinqh_gemv_noalloc(dl.L, xd, td, dl.planes, dl.s, dl.z, yb_na)
        torch.cuda.synchronize()
        ref = C.gemv(x, theta, q, s, z, b_max)
        a, b = y_ws.cpu().numpy().astype(np.float64), y_na.cpu().numpy().astype(np.float64)
        assert O.max_rel_error(b, ref) <= TOL_F32
        if exact:
            assert np.array_equal(a, ref) and np.array_equal(b, a)
            want = O.round_to_bf16(ref.astype(np.float32))
            assert np.array_equal(yb_na.view(torch.int16).cpu().numpy().view(np.uint16), want)
        else:
            assert O.max_rel_error(b, a) <= 5e-4


def test_gemv_noalloc_rejects_layout_beyond_scratch(dev):
    """A layer whose workspace exceeds the static array is refused with
    GRINQH_ENOSPACE before anything is launched; the workspace call accepts it."""
    import torch
    import input_adaptive_bit_amd as G
    L = G.grinqh_layout_init(64, 1 << 20, 8)
    assert G.grinqh_gemv_workspace_bytes(L) > G.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(64, dtype=torch.bfloat16, device=dev)
    th = torch.zeros(4, dtype=torch.float32, device=dev)
    planes = torch.zeros(G.grinqh_packed_bytes(L) // 4, dtype=torch.int32, device=dev)
    s = torch.zeros(1 << 20, dtype=torch.float16, device=dev)
    z = torch.zeros(1 << 20, dtype=torch.float16, device=dev)
    y = torch.empty(1 << 20, dtype=torch.float32, device=dev)
    with pytest.raises(G.GrinqhError) as e:
        G.grinqh_gemv_noalloc(L, x, th, planes, s, z, y)
    assert e.value.status == 3          # GRINQH_ENOSPACE
