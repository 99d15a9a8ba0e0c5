"""GPU parity of grouped GEMV launches (grinqh_gemv_group, through the C
ABI): each member of a launch of differently shaped GEMVs against the fp64
oracle and against the single-GEMV call on the same inputs."""

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


def _theta_dev(theta, dev):
    return to_dev(np.asarray(theta, np.float32), dev)


def _mismatch(got, ref, n=8):
    """The outputs that differ most from the reference: (index, got, ref)."""
    got = np.asarray(got, np.float64)
    d = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-2 * np.sqrt(np.mean(ref ** 2)))
    idx = np.argsort(-d)[:n]
    return [(int(j), float(got[j]), float(ref[j])) for j in idx]


@pytest.mark.parametrize("b_max,x_dtype", [(8, "bf16"), (4, "bf16"), (8, "f32")])
def test_gemv_group_matches_oracle_and_single_calls(dev, b_max, x_dtype):
    """A group launch of differently shaped members: each member matches the
    oracle and the single-GEMV call on the same inputs."""
    import torch
    import input_adaptive_bit_amd as G
    shapes = [(4096, 4096), (4096, 1024), (4096, 14336), (14336, 4096), (300, 1500), (1, 65)]
    rng = np.random.default_rng(77 + b_max)
    members, ops, refs, singles = [], [], [], []
    say(f"group launch b_max={b_max} x={x_dtype} members={len(shapes)}")
    for di, do in shapes:
        q = rng.integers(0, 1 << b_max, size=(do, di), dtype=np.uint8)
        s = rng.uniform(0.001, 0.01, do).astype(np.float16)
        z = rng.normal(0, 0.01, do).astype(np.float16)
        x = rng.standard_t(3, di).astype(np.float32)
        if x_dtype == "bf16":
            x = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
        theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
        dl = DeviceLinear(q, s, z, b_max, dev)
        xd, td = to_dev_x(x, x_dtype, dev), _theta_dev(theta, dev)
        y = torch.empty(do, dtype=torch.float32, device=dev)
        members.append(dl)
        ops.append((xd, td, dl.planes, dl.s, dl.z, y))
        refs.append(C.gemv(x, theta, q, s, z, b_max))
        singles.append(dl.gemv(xd, td, torch.float32))
    torch.cuda.synchronize()
    for k, (single, ref) in enumerate(zip(singles, refs)):
        assert O.max_rel_error(single.cpu().numpy(), ref) <= TOL_F32, ("single", k)
    layouts = [m.L for m in members]
    ws = G.new_group_workspace(layouts, dev)
    for rep in range(3):
        for o in ops:
            o[5].fill_(float("nan"))
        G.grinqh_gemv_group(layouts, ops, ws)
        torch.cuda.synchronize()
        for k, (o, ref, single) in enumerate(zip(ops, refs, singles)):
            got = o[5].cpu().numpy()
            err = O.max_rel_error(got, ref)
            sg = single.cpu().numpy()
            assert err <= TOL_F32, (rep, k, err, _mismatch(got, ref))
            assert O.max_rel_error(got, sg) <= 5e-4, (rep, k, _mismatch(got, sg))
