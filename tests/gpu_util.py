"""Helpers for the GPU parity tests: move seeded inputs to the device, run
the HIP path through the C ABI (the binding), and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np

TOL_F32 = 2e-3                 # max relative error of fp32 y vs the fp64 oracle
TOL_BF16 = 2e-3 + 2.0 ** -8    # bf16 y adds at most one bf16 rounding (2^-8 relative)


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X (no CPU fallback)")
    return torch.device("cuda:0")


def to_dev_x(x_f32, x_dtype, dev):
    import torch
    import synthetic as S
    if x_dtype == "bf16":
        bits = S.f32_to_bf16_bits(np.asarray(x_f32, np.float32))
        return torch.from_numpy(bits.view(np.int16).copy()).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x_f32, np.float32)).to(dev)


def to_dev(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class DeviceLinear:
    """One linear layer resident on the device, packed by the HIP library."""

    def __init__(self, q, s, z, b_max, dev, q_dev=None):
        import input_adaptive_bit_amd as G
        import torch
        self.b_max = b_max
        self.q_np = None if q is None else np.asarray(q, np.uint8)
        self.s_np = np.asarray(s, np.float16)
        self.z_np = np.asarray(z, np.float16)
        self.q_dev = q_dev if q_dev is not None else to_dev(q, dev)
        self.d_out, self.d_in = self.q_dev.shape
        self.L, self.planes = G.pack(self.q_dev, b_max)
        self.s = to_dev(np.asarray(s, np.float16), dev)
        self.z = to_dev(np.asarray(z, np.float16), dev)
        self.ws = G.new_workspace(self.L, dev)
        self.dev = dev
        torch.cuda.synchronize()

    def gemv(self, x_dev, theta_dev, out_dtype=None):
        import input_adaptive_bit_amd as G
        return G.gemv(self.L, x_dev, theta_dev, self.planes, self.s, self.z, self.ws, out_dtype)

    def planes_np(self):
        return self.planes.cpu().numpy().view(np.uint32)
