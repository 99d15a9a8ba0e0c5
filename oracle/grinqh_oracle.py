"""Plain fp64 CPU oracle for the GRINQH batch-1 decode GEMV.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this module.  The HIP library never calls it,
and this module never calls the HIP library: the two share no code.

Source: the page "GRINQH: Graded Input-Based Quantization Hierarchy for
Efficient LLM Generation" (papernotes.org note on arXiv 2606.23419).  In the
citations below, "KD1", "KD2" and "KD3" are items 1-3 of that page's
方法详解 / 关键设计 (key design) section:

* KD1 - activation-graded precision mapping: the bit-assignment equation;
* KD2 - nested bit-planar storage and sparse loading;
* KD3 - midpoint truncation-bias correction: the dequantisation equation.

Readings taken where the page is silent or garbled (each is also listed with
its reason in the design notes):

* Thresholds.  There are P = b_max/2 ascending thresholds theta_1..theta_P
  and P+1 levels {0, 2, ..., b_max}; b_i = 2 * #{k : theta_k <= |x_i|}.
  A tie |x_i| = theta_k goes to the upper level (half-open intervals in the
  KD1 equation).  NaN compares false everywhere -> 0 bits; +-Inf -> b_max.
* Planes.  Plane p (p = 0 most significant) holds bits
  [b_max-2p-2, b_max-2p-1] of q (KD2: 2-bit fragments stacked from high to
  low significance).  Layout planes[i][p][w] (channel-major, reduction
  dimension first, so a channel's taken planes are one contiguous prefix),
  W_row = ceil(d_out/64)*4 words per plane row, fragment of output 16w+t at
  bits [2t, 2t+1] of word w (KD2: 16 fragments per uint32), padding
  fragments 0.
* Truncation and phi.  q_b * 2^(b_max-b) = (q >> k) << k with k = b_max - b
  (KD3: the spliced truncated integer), and phi = 2^(k-1), also at
  k = 0 (phi = 1/2; KD3 gives no exception).  A channel with b = 0
  contributes nothing (KD1: its weights are never loaded).
* s and z are per output channel (fp16), widened exactly to fp64.
* Threshold calibration (KD1 calibrates the thresholds offline on the
  magnitudes of about 128 sample inputs).  The magnitudes |x| of all samples
  are pooled and sorted ascending (NaN after +Inf); the threshold at level q
  is the linear-interpolation quantile v[lo] + t * (v[hi] - v[lo]) with
  h = (n - 1) * q, lo = floor(h), hi = min(lo + 1, n - 1), t = h - lo,
  computed in fp64 and rounded once to fp32; at t = 0 it is v[lo] itself.
* Offline quantisation ("RTN", named by the page as a base the method can
  sit on, not defined there).  Per output channel j, asymmetric
  round-to-nearest onto the b_max-bit grid of interval midpoints that the
  KD3 dequantisation reconstructs at b = b_max: lo_j and hi_j are the row's
  minimum and maximum (NaN ignored), s_j = fp16((hi_j - lo_j) / 2^b_max),
  z_j = fp16(lo_j) (a zero stored as +0), and q = min(max(floor((w - z_j) / s_j), 0), 2^b_max - 1)
  in fp32 with the stored s_j and z_j (a NaN quotient gives 0; a row with
  s_j = 0 gets q = 0).  Then s_j * (q + 1/2) + z_j is the midpoint of w's
  interval, within s_j / 2 of w.

* Prefill (the overview: dense b_max weights in the prefill stage, whose
  19-20% slowdown the page puts down to unpacking).  Every channel is taken at
  b = b_max whatever its activation: Y = X * W_hat^T with the KD3 weights at
  k = 0, phi = 1/2.

Parity pins that hold this module to the page and to mathematics are in
tests/test_oracle_pins.py; none of them retypes the formulas below.
"""

from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "n_planes", "row_words", "assign_bits", "active_channels", "pack_planes",
    "unpack_fragments", "truncated_codes", "codes_from_planes", "phi",
    "dequant", "gemv", "gemv_from_planes", "gemv_columns", "eff_bits",
    "required_bytes", "bias_table", "round_to_bf16", "max_rel_error",
    "quantile_position", "calibrate_thresholds", "quantize_rtn",
]


def n_planes(b_max: int) -> int:
    if b_max not in (2, 4, 6, 8):
        raise ValueError("b_max must be 2, 4, 6 or 8")
    return b_max // 2


def row_words(d_out: int) -> int:
    """uint32 words per plane row: d_out padded to a multiple of 64 outputs."""
    return ((d_out + 63) // 64) * 4


# --------------------------------------------------------------------------
# KD1: bit assignment
# --------------------------------------------------------------------------

def assign_bits(x, theta, b_max: int) -> np.ndarray:
    """b_i = b_k for |x_i| in [theta_k, theta_{k+1}), theta_0 = 0, last = inf.

    Counting the thresholds at or below |x_i| is the same interval test for
    ascending thresholds.  Inputs are the exact fp32/bf16 values widened to
    fp64, so every comparison has the same outcome as in fp32.
    """
    P = n_planes(b_max)
    a = np.abs(np.asarray(x, dtype=np.float64))
    th = np.asarray(theta, dtype=np.float64)
    if th.shape != (P,):
        raise ValueError(f"need {P} thresholds for b_max={b_max}")
    level = np.zeros(a.shape, dtype=np.int64)
    for k in range(P):
        level += (th[k] <= a)          # NaN compares false -> stays 0
    return (2 * level).astype(np.uint8)


def active_channels(bits) -> np.ndarray:
    """Ascending indices of channels with b_i > 0 (the channels that are loaded)."""
    return np.nonzero(np.asarray(bits) > 0)[0].astype(np.int32)


# --------------------------------------------------------------------------
# KD2: bit-planar, reduction-dim-major storage
# --------------------------------------------------------------------------

def pack_planes(q, b_max: int) -> np.ndarray:
    """q uint8 [d_out][d_in] -> planes uint32 [d_in][P][W_row]."""
    P = n_planes(b_max)
    q = np.asarray(q, dtype=np.uint8)
    d_out, d_in = q.shape
    W = row_words(d_out)
    qt = (q.T.astype(np.uint32)) & ((1 << b_max) - 1)          # [d_in][d_out]
    padded = np.zeros((d_in, W * 16), dtype=np.uint32)
    padded[:, :d_out] = qt
    planes = np.zeros((d_in, P, W), dtype=np.uint32)
    for p in range(P):
        frag = (padded >> (b_max - 2 * p - 2)) & 3                 # [d_in][W*16]
        frag = frag.reshape(d_in, W, 16)
        word = np.zeros((d_in, W), dtype=np.uint32)
        for t in range(16):
            word |= frag[:, :, t] << (2 * t)
        planes[:, p, :] = word
    return planes


def unpack_fragments(planes, d_out: int) -> np.ndarray:
    """planes [d_in][P][W] -> fragments uint8 [d_in][P][d_out]."""
    planes = np.asarray(planes, dtype=np.uint32)
    d_in, P, W = planes.shape
    t = np.arange(16, dtype=np.uint32)
    frag = (planes[:, :, :, None] >> (2 * t)) & 3                  # [d_in][P][W][16]
    return frag.reshape(d_in, P, W * 16)[:, :, :d_out].astype(np.uint8)


# --------------------------------------------------------------------------
# KD3: truncation, midpoint bias, dequantisation
# --------------------------------------------------------------------------

def truncated_codes(q, bits, b_max: int) -> np.ndarray:
    """codes[..., i, j] = (q[j][i] >> k_i) << k_i for active i, 0 otherwise.

    ``bits`` may carry leading batch dimensions ([..., d_in]).
    """
    q = np.asarray(q, dtype=np.int64)                              # [d_out][d_in]
    bits = np.asarray(bits, dtype=np.int64)
    k = (b_max - bits)[..., :, None]                               # [..., d_in, 1]
    qt = q.T & ((1 << b_max) - 1)                                  # [d_in][d_out]
    c = (qt >> k) << k
    return np.where(bits[..., :, None] > 0, c, 0)


def codes_from_planes(planes, bits, b_max: int, d_out: int) -> np.ndarray:
    """Sum of the taken planes' fragments at their significance (KD2 + KD3)."""
    P = n_planes(b_max)
    frag = unpack_fragments(planes, d_out).astype(np.int64)        # [d_in][P][d_out]
    bits = np.asarray(bits, dtype=np.int64)
    taken = bits // 2
    codes = np.zeros((frag.shape[0], d_out), dtype=np.int64)
    for p in range(P):
        use = (p < taken)[:, None]
        codes += np.where(use, frag[:, p, :] * (4 ** (P - 1 - p)), 0)
    return codes


def phi(bits, b_max: int) -> np.ndarray:
    """phi_i = 2^(b_max - b_i - 1); 0 for skipped channels (no weight at all)."""
    bits = np.asarray(bits, dtype=np.int64)
    k = b_max - bits
    return np.where(bits > 0, np.ldexp(1.0, k - 1), 0.0)


def dequant(codes, bits, s, z, b_max: int) -> np.ndarray:
    """w_hat[..., i, j] = s_j * (codes_ij + phi_i) + z_j for active i, else 0."""
    codes = np.asarray(codes, dtype=np.float64)
    bits = np.asarray(bits)
    s = np.asarray(s, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    ph = phi(bits, b_max)[..., :, None]
    w = s * (codes + ph) + z
    return np.where(np.asarray(bits)[..., :, None] > 0, w, 0.0)


def gemv(x, theta, q, s, z, b_max: int, exact: bool = False) -> np.ndarray:
    """y_j = sum over active i of x_i * w_hat_ij, in fp64.

    ``x`` may be [d_in] or a batch [n][d_in] (each row its own decode step).
    ``exact`` sums each output with math.fsum (small inputs only).
    """
    x = np.asarray(x, dtype=np.float64)
    bits = assign_bits(x, theta, b_max)
    codes = truncated_codes(q, bits, b_max)
    w = dequant(codes, bits, s, z, b_max)                          # [..., d_in, d_out]
    xs = np.where(bits > 0, x, 0.0)          # skipped channels: no term at all
    if exact:
        if x.ndim != 1:
            raise ValueError("exact summation takes one vector")
        return np.array([math.fsum(xs * w[:, j]) for j in range(w.shape[1])])
    return np.einsum("...i,...ij->...j", xs, w)


def gemv_from_planes(x, theta, planes, s, z, b_max: int, d_out: int) -> np.ndarray:
    """Same product, with the codes read back from the packed planes."""
    x = np.asarray(x, dtype=np.float64)
    bits = assign_bits(x, theta, b_max)
    codes = codes_from_planes(planes, bits, b_max, d_out)
    w = dequant(codes, bits, s, z, b_max)
    xs = np.where(bits > 0, x, 0.0)
    return xs @ w


def gemv_columns(x, theta, q_rows, s_cols, z_cols, b_max: int) -> np.ndarray:
    """Outputs for a sample of output channels: q_rows is q[cols, :]."""
    return gemv(x, theta, q_rows, s_cols, z_cols, b_max)


# --------------------------------------------------------------------------
# Prefill stage: the dense b_max dequant GEMM
# --------------------------------------------------------------------------

def prefill_gemm(X, q, s, z, b_max: int) -> np.ndarray:
    """Y[m][j] = sum_i X[m][i] * w_hat_ij with every channel at b = b_max, in fp64.

    The page's overview keeps the prefill stage dense: all weights at b_max
    precision in ordinary matrix products, no thresholds.  With b = b_max for
    every channel KD3 gives k = 0 and phi = 1/2, so w_hat_ij = s_j * (q_ji +
    1/2) + z_j on the whole b_max-bit code.  X is [M][d_in] (M prompt tokens),
    Y is [M][d_out].
    """
    X = np.asarray(X, dtype=np.float64)
    full = np.full(X.shape[-1], b_max, dtype=np.int64)
    w = dequant(truncated_codes(q, full, b_max), full, s, z, b_max)     # [d_in][d_out]
    return X @ w


# --------------------------------------------------------------------------
# KD1: threshold calibration (offline)
# --------------------------------------------------------------------------

def quantile_position(n: int, level: float):
    """Where level q falls among n sorted values: (lo, hi, t) with
    h = (n - 1) * q in fp64, lo = floor(h), hi = min(lo + 1, n - 1), t = h - lo."""
    if n < 1:
        raise ValueError("no values")
    if not (0.0 <= level <= 1.0):
        raise ValueError("quantile level outside [0, 1]")
    h = float(n - 1) * float(level)
    lo = int(math.floor(h))
    hi = min(lo + 1, n - 1)
    return lo, hi, h - lo


def calibrate_thresholds(x_calib, levels) -> np.ndarray:
    """KD1: the thresholds as quantiles of the pooled calibration magnitudes
    (see the reading in the module notes).  x_calib: any shape, fp32 values
    (bf16 inputs widened exactly); levels: one per threshold, in [0, 1]."""
    mags = np.abs(np.asarray(x_calib, dtype=np.float32).ravel()).astype(np.float64)
    v = np.sort(mags)                      # ascending, NaN last
    out = np.empty(len(levels), dtype=np.float64)
    for k, q in enumerate(levels):
        lo, hi, t = quantile_position(v.size, q)
        a, b = v[lo], v[hi]
        # two roundings in fp64, no fused multiply-add; a level that falls on
        # a value (t = 0) returns that value, even next to an infinite one
        out[k] = a if t == 0.0 else a + t * (b - a)
    return out.astype(np.float32)


# --------------------------------------------------------------------------
# Offline quantisation front end (RTN onto the KD3 midpoint grid)
# --------------------------------------------------------------------------

def quantize_rtn(w, b_max: int):
    """Codes, scales and zero points of a weight matrix w [d_out][d_in]
    (fp32 values, e.g. widened from bf16) at b_max bits; see the reading in
    the module notes.  Returns (q uint8 [d_out][d_in], s fp16 [d_out],
    z fp16 [d_out]).  All arithmetic in fp32, as the reading fixes it."""
    w = np.asarray(w, dtype=np.float32)
    levels = np.float32(1 << b_max)
    lo = np.fmin.reduce(w, axis=1)                     # NaN ignored
    hi = np.fmax.reduce(w, axis=1)
    # "+ 0" turns a -0 into +0, so the stored s and z have one zero
    s = ((hi - lo) / levels + np.float32(0)).astype(np.float16)
    z = (lo + np.float32(0)).astype(np.float16)
    s32 = s.astype(np.float32)[:, None]
    z32 = z.astype(np.float32)[:, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        u = np.floor((w - z32) / s32)
    u = np.where(np.isnan(u), np.float32(0), u)
    u = np.minimum(np.maximum(u, np.float32(0)), levels - np.float32(1))
    u = np.where(s32 == 0, np.float32(0), u)
    return u.astype(np.uint8), s, z


# --------------------------------------------------------------------------
# Measurement definitions
# --------------------------------------------------------------------------

def eff_bits(bits) -> float:
    """Effective bits of one GEMV: the mean assigned width over input channels."""
    return float(np.mean(np.asarray(bits, dtype=np.float64)))


def required_bytes(bits, d_out: int) -> Dict[str, float]:
    """Bytes the decode path must move: taken planes plus fp16 s and z."""
    plane_bits = float(np.sum(np.asarray(bits, dtype=np.float64))) * d_out
    planes = plane_bits / 8.0
    return {"planes": planes, "scales": 4.0 * d_out, "total": planes + 4.0 * d_out}


def bias_table(b_max: int, s: float = 1.0, z: float = 0.0) -> Dict[int, Dict[str, float]]:
    """Mean reconstruction offsets over all codes q in [0, 2^b_max), per width b.

    * ``midpoint_vs_full``: mean of w_hat_b(q) - w_hat_bmax(q), both with phi;
    * ``floor_vs_exact``: mean of (s*((q>>k)<<k) + z) - (s*q + z), no phi;
    * ``midpoint_vs_exact``: mean of w_hat_b(q) - (s*q + z).
    """
    q = np.arange(1 << b_max, dtype=np.int64)
    out = {}
    full_bits = np.full(1, b_max)
    w_full = dequant(truncated_codes(q[:, None], full_bits, b_max), full_bits,
                     [s] * q.size, [z] * q.size, b_max)[0]
    for b in range(2, b_max + 1, 2):
        bits = np.full(1, b)
        codes = truncated_codes(q[:, None], bits, b_max)[0]        # [q]
        w_b = dequant(codes[None, :], bits, [s] * q.size, [z] * q.size, b_max)[0]
        floor_rec = s * codes.astype(np.float64) + z
        exact = s * q.astype(np.float64) + z
        out[b] = {
            "midpoint_vs_full": float(np.mean(w_b - w_full)),
            "floor_vs_exact": float(np.mean(floor_rec - exact)),
            "midpoint_vs_exact": float(np.mean(w_b - exact)),
        }
    return out


# --------------------------------------------------------------------------
# Checking helpers
# --------------------------------------------------------------------------

def round_to_bf16(y32) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (NaN kept NaN)."""
    y32 = np.ascontiguousarray(y32, dtype=np.float32)
    u = y32.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(y32)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def max_rel_error(y, y_ref, floor_frac: float = 1e-2) -> float:
    """max_j |y_j - y*_j| / max(|y*_j|, floor_frac * rms(y*))."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    denom = np.maximum(np.abs(y_ref), floor_frac * rms)
    denom = np.where(denom > 0, denom, 1.0)
    if y.size == 0:
        return 0.0
    return float(np.max(np.abs(y - y_ref) / denom))
