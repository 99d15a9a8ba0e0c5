"""Seeded synthetic workloads for the batch-1 decode GEMV.

Every array is drawn from ``numpy.random.default_rng([2026, cfg, shape, layer,
linear, role])`` so that any one piece can be regenerated on its own.  Roles:

* 0 - weight codes q, uint8 [d_out][d_in], uniform over [0, 2**b_max)
* 1 - per-output scale s, U(0.001, 0.01) rounded to fp16
* 2 - per-output zero point z, N(0, sd=0.01) rounded to fp16
* 3 - the permutation that picks the persistent outlier channels
* 4 - the activation stream: 128 calibration vectors, then the test vector
* 10 + c - the weight codes of the c-th extra copy used to defeat caches

The activations stand in for real decode-time inputs of Llama-3.1-8B- and
70B-shaped linear layers (heavy tails, a few persistent outlier channels);
no model weights or text are used.  The thresholds are the harness's
stand-in for the offline calibration of the GRINQH note (key design 1:
quantiles of |x| over about 128 samples): pooled |x| of the 128 calibration
vectors, ``numpy.quantile`` (linear) in fp64, then rounded to fp32.

bf16 activations are produced by round-to-nearest-even from fp32 and carried
as their uint16 bit patterns next to an fp32 array holding the same values.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "LinearSpec", "Linear", "QUANTILES_B8", "QUANTILES_B6", "QUANTILES_B4", "QUANTILES_SMALL",
    "rng_for", "f32_to_bf16_bits", "bf16_bits_to_f32", "fp16_bits",
    "gen_codes", "gen_scales", "gen_x_stream", "calibrate_theta", "make_linear",
    "small_case", "llama8b_linears", "llama8b_linears_b6", "llama8b_linears_b4", "llama8b_decode_step",
    "llama70b_linears", "LLAMA8B_SHAPES", "LLAMA8B_FUSED_LAYER", "LLAMA8B_LAYER_UNFUSED", "LLAMA70B_SHAPES",
    "llama8b_decode_step_unfused",
    "torch_seed",
]

# Cumulative |x| quantile levels (one per threshold).  With the level shares
# they imply, the expected mean bit width is exactly the key of each table.
QUANTILES_B8 = {
    2: (0.38, 0.73, 0.92, 0.97),   # shares 38/35/19/5/3 % of 0/2/4/6/8 bits
    3: (0.20, 0.52, 0.82, 0.96),   # 20/32/30/14/4
    4: (0.10, 0.35, 0.65, 0.90),   # 10/25/30/25/10
    6: (0.05, 0.10, 0.25, 0.60),   # 5/5/15/35/40
    8: None,                       # dense: every threshold 0 -> all b_max
}
QUANTILES_B6 = {
    2: (0.30, 0.75, 0.95),         # shares 30/45/20/5 % of 0/2/4/6 bits
    3: (0.20, 0.50, 0.80),         # 20/30/30/20
    4: (0.10, 0.30, 0.60),         # 10/20/30/40
    6: None,                       # dense
}
QUANTILES_B4 = {
    1.5: (0.40, 0.85),             # 40/45/15 % of 0/2/4 bits
    2: (0.30, 0.70),
    3: (0.10, 0.40),
    4: None,                       # dense
}
QUANTILES_SMALL = (0.20, 0.50, 0.80, 0.95)   # 20/30/30/15/5 %, mean ~3.1 bits

LLAMA8B_SHAPES = ((4096, 4096), (4096, 14336), (14336, 4096))
# one decoder layer as decode launches it (d_in, d_out): q, k and v read the same
# x and run as one fused q|k|v projection, gate and up likewise as gate|up;
# o needs the attention output and down the activated gate|up output, so the
# four run one after another
LLAMA8B_FUSED_LAYER = ((4096, 6144), (4096, 4096), (4096, 28672), (14336, 4096))
# the same layer as its seven separate linears (d_in, d_out, input group): q, k and
# v share one input, gate and up another
LLAMA8B_LAYER_UNFUSED = ((4096, 4096, 0), (4096, 1024, 0), (4096, 1024, 0), (4096, 4096, 1),
                         (4096, 14336, 2), (4096, 14336, 2), (14336, 4096, 3))
LLAMA70B_SHAPES = ((8192, 8192), (8192, 28672), (28672, 8192))


@dataclasses.dataclass(frozen=True)
class LinearSpec:
    d_in: int
    d_out: int
    b_max: int
    x_kind: str                      # "normal" or "t3"
    x_dtype: str                     # "f32" or "bf16"
    quantiles: Optional[Tuple[float, ...]]   # None -> dense (all thresholds 0)
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0
    key: Tuple[int, int, int, int] = (0, 0, 0, 0)   # (cfg, shape, layer, linear)
    n_calib: int = 128


@dataclasses.dataclass
class Linear:
    spec: LinearSpec
    q: np.ndarray            # uint8 [d_out][d_in]
    s: np.ndarray            # float16 [d_out]
    z: np.ndarray            # float16 [d_out]
    x: np.ndarray            # float32 [d_in]   (values exactly representable in x_dtype)
    x_bits: Optional[np.ndarray]  # uint16 [d_in] bf16 patterns when x_dtype == "bf16"
    theta: np.ndarray        # float32 [b_max // 2]
    outliers: np.ndarray     # int64 channel indices


def rng_for(key: Sequence[int], role: int) -> np.random.Generator:
    return np.random.default_rng([2026, *[int(k) for k in key], int(role)])


def torch_seed(key: Sequence[int], role: int) -> int:
    """A 63-bit seed for torch generators, derived from the same key/role."""
    ss = np.random.SeedSequence([2026, *[int(k) for k in key], int(role)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); NaN stays a quiet NaN."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    out = rounded.astype(np.uint16)
    out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def fp16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float16).view(np.uint16)


def gen_codes(spec: LinearSpec, role: int = 0) -> np.ndarray:
    rng = rng_for(spec.key, role)
    return rng.integers(0, 1 << spec.b_max, size=(spec.d_out, spec.d_in), dtype=np.uint8)


def gen_scales(spec: LinearSpec) -> Tuple[np.ndarray, np.ndarray]:
    s = rng_for(spec.key, 1).uniform(0.001, 0.01, size=spec.d_out).astype(np.float16)
    z = rng_for(spec.key, 2).normal(0.0, 0.01, size=spec.d_out).astype(np.float16)
    return s, z


def _outlier_channels(spec: LinearSpec) -> np.ndarray:
    n = int(np.floor(spec.outlier_frac * spec.d_in))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    return np.sort(rng_for(spec.key, 3).permutation(spec.d_in)[:n]).astype(np.int64)


def gen_x_stream(spec: LinearSpec) -> Tuple[np.ndarray, np.ndarray]:
    """(n_calib + 1) activation vectors as fp32 values of the x dtype, and the outliers."""
    rng = rng_for(spec.key, 4)
    shape = (spec.n_calib + 1, spec.d_in)
    if spec.x_kind == "normal":
        xs = rng.standard_normal(shape)
    elif spec.x_kind == "t3":
        xs = rng.standard_t(3, size=shape)
    else:
        raise ValueError(f"unknown x_kind {spec.x_kind!r}")
    outl = _outlier_channels(spec)
    if outl.size:
        xs[:, outl] *= spec.outlier_scale
    xs = xs.astype(np.float32)
    if spec.x_dtype == "bf16":
        xs = bf16_bits_to_f32(f32_to_bf16_bits(xs)).reshape(shape)
    elif spec.x_dtype != "f32":
        raise ValueError(f"unknown x_dtype {spec.x_dtype!r}")
    return xs, outl


def calibrate_theta(x_calib: np.ndarray, quantiles: Optional[Sequence[float]],
                    n_thresholds: int) -> np.ndarray:
    if quantiles is None:
        return np.zeros(n_thresholds, dtype=np.float32)
    if len(quantiles) != n_thresholds:
        raise ValueError("one quantile level per threshold")
    pooled = np.abs(np.asarray(x_calib, dtype=np.float64)).ravel()
    return np.quantile(pooled, np.asarray(quantiles, dtype=np.float64)).astype(np.float32)


def make_linear(spec: LinearSpec, with_codes: bool = True) -> Linear:
    xs, outl = gen_x_stream(spec)
    theta = calibrate_theta(xs[: spec.n_calib], spec.quantiles, spec.b_max // 2)
    x = np.ascontiguousarray(xs[spec.n_calib])
    x_bits = f32_to_bf16_bits(x) if spec.x_dtype == "bf16" else None
    s, z = gen_scales(spec)
    q = gen_codes(spec) if with_codes else None
    return Linear(spec=spec, q=q, s=s, z=z, x=x, x_bits=x_bits, theta=theta, outliers=outl)


# ---------------------------------------------------------------------------
# The workloads.  cfg ids 1..5 only feed the seeds.
# ---------------------------------------------------------------------------

def small_case() -> LinearSpec:
    """1024 -> 1024, b_max 8, fp32 x ~ N(0,1) with 1 % of channels x20."""
    return LinearSpec(1024, 1024, 8, "normal", "f32", QUANTILES_SMALL,
                      outlier_frac=0.01, outlier_scale=20.0, key=(1, 0, 0, 0))


def llama8b_linears(eff_bits: int) -> list:
    """Attention projection and MLP shapes of an 8B Llama, b_max 8, bf16 x ~ t(3)."""
    return [LinearSpec(di, do, 8, "t3", "bf16", QUANTILES_B8[eff_bits], key=(2, k, 0, 0))
            for k, (di, do) in enumerate(LLAMA8B_SHAPES)]


def llama8b_linears_b6(eff_bits: int) -> list:
    """Same shapes with b_max 6 (levels 0/2/4/6); bf16 x ~ t(3)."""
    return [LinearSpec(di, do, 6, "t3", "bf16", QUANTILES_B6[eff_bits], key=(7, k, 0, 0))
            for k, (di, do) in enumerate(LLAMA8B_SHAPES)]


def llama8b_linears_b4(eff_bits: float) -> list:
    """Same shapes with b_max 4; bf16 x ~ N(0,1) with 0.5 % of channels x30."""
    return [LinearSpec(di, do, 4, "normal", "bf16", QUANTILES_B4[eff_bits],
                       outlier_frac=0.005, outlier_scale=30.0, key=(3, k, 0, 0))
            for k, (di, do) in enumerate(LLAMA8B_SHAPES)]


def llama8b_decode_step(eff_bits: int, n_layers: int = 32) -> list:
    """The projections of every decoder layer in launch order (fused q|k|v, o,
    fused gate|up, down), each with its own x and thresholds; a fused
    projection has one x and one threshold vector."""
    out = []
    for layer in range(n_layers):
        for lin, (di, do) in enumerate(LLAMA8B_FUSED_LAYER):
            out.append(LinearSpec(di, do, 8, "t3", "bf16", QUANTILES_B8[eff_bits],
                                  key=(4, 1, layer, lin)))
    return out


def llama8b_decode_step_unfused(eff_bits: int, n_layers: int = 32) -> list:
    """The seven linears of every decoder layer as separate launches, in
    order (q, k, v, o, gate, up, down): (spec, input key) pairs, where
    linears of one layer with the same input key read the same x and
    thresholds (those of the first of them)."""
    out = []
    for layer in range(n_layers):
        for lin, (di, do, grp) in enumerate(LLAMA8B_LAYER_UNFUSED):
            out.append((LinearSpec(di, do, 8, "t3", "bf16", QUANTILES_B8[eff_bits], key=(4, 3, layer, lin)),
                        (layer, grp)))
    return out


def llama70b_linears(eff_bits: int) -> list:
    return [LinearSpec(di, do, 8, "t3", "bf16", QUANTILES_B8[eff_bits], key=(5, k, 0, 0))
            for k, (di, do) in enumerate(LLAMA70B_SHAPES)]
