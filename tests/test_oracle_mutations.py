"""Plant plausible mistakes in the CPU oracle and check that the pins catch each.

Every mutation is applied to the oracle module on the CPU (monkeypatch) and
undone afterwards; the HIP library is not involved.
"""

import numpy as np
import pytest

from oracle import grinqh_oracle as O
import tests.test_oracle_pins as pins


def _pins(golden_dir):
    return [
        lambda: pins.test_assign_bits_golden_ties(golden_dir),
        lambda: pins.test_assign_bits_is_searchsorted(8),
        lambda: pins.test_pack_golden_hand_examples(golden_dir),
        lambda: pins.test_codes_exhaustive(8),
        lambda: pins.test_midpoint_is_interval_centroid(4),
        lambda: pins.test_bias_table_closed_forms(golden_dir),
        lambda: pins.test_tiny_gemv_golden(golden_dir),
        lambda: pins.test_dense_mode_is_plain_dot(8),
        lambda: pins.test_single_active_channel(),
        lambda: pins.test_factorised_form(4),
        lambda: pins.test_calibration_matches_numpy_linear_quantile(1000),
        lambda: pins.test_calibration_closed_forms(),
        lambda: pins.test_calibration_ties_and_nan_order(),
        lambda: pins.test_rtn_codes_on_an_exact_integer_grid(3),
        lambda: pins.test_rtn_codes_at_interval_centres(),
        lambda: pins.test_rtn_round_trip_bound(8),
        lambda: pins.test_rtn_special_rows(),
        lambda: pins.test_prefill_integer_exact(),
        lambda: pins.test_prefill_constant_codes_closed_form(),
        lambda: pins.test_prefill_of_rtn_weights_approximates_the_weights(),
    ]


def _mut_phi_exponent(bits, b_max):
    bits = np.asarray(bits, dtype=np.int64)
    return np.where(bits > 0, np.ldexp(1.0, b_max - bits), 0.0)


def _mut_phi_zero_at_full(bits, b_max):
    bits = np.asarray(bits, dtype=np.int64)
    k = b_max - bits
    return np.where((bits > 0) & (k > 0), np.ldexp(1.0, k - 1), 0.0)


_orig_assign = O.assign_bits
_orig_pack = O.pack_planes
_orig_dequant = O.dequant
_orig_trunc = O.truncated_codes


def _mut_ties_down(x, theta, b_max):
    a = np.abs(np.asarray(x, dtype=np.float64))
    level = sum((np.float64(t) < a).astype(np.int64) for t in np.asarray(theta, np.float64))
    return (2 * level).astype(np.uint8)


def _mut_planes_lsb_first(q, b_max):
    return _orig_pack(q, b_max)[:, ::-1, :].copy()


def _mut_word_order_reversed(q, b_max):
    planes = _orig_pack(q, b_max)
    out = np.zeros_like(planes)
    for t in range(16):
        out |= ((planes >> (2 * t)) & 3) << (2 * (15 - t))
    return out


def _mut_drop_z(codes, bits, s, z, b_max):
    return _orig_dequant(codes, bits, s, np.zeros_like(np.asarray(z, dtype=np.float64)), b_max)


def _mut_round_not_truncate(q, bits, b_max):
    q = np.asarray(q, dtype=np.int64)
    bits = np.asarray(bits, dtype=np.int64)
    k = (b_max - bits)[..., :, None]
    qt = q.T
    c = np.minimum(((qt + ((1 << k) >> 1)) >> k) << k, (1 << b_max) - 1)
    return np.where(bits[..., :, None] > 0, c, 0)


def _mut_level_count_off_by_one(x, theta, b_max):
    b = _orig_assign(x, theta, b_max).astype(np.int64)
    return np.minimum(b + 2 * (b > 0), b_max).astype(np.uint8)


_orig_qpos = O.quantile_position
_orig_calib = O.calibrate_thresholds


def _mut_quantile_index_n(n, level):
    h = min(float(n) * float(level), float(n - 1))
    lo = int(np.floor(h))
    return lo, min(lo + 1, n - 1), h - lo


def _mut_quantile_no_interpolation(n, level):
    lo, hi, t = _orig_qpos(n, level)
    return lo, hi, 0.0


def _mut_calibration_signed(x_calib, levels):
    v = np.sort(np.asarray(x_calib, dtype=np.float64).ravel())
    out = []
    for q in levels:
        lo, hi, t = _orig_qpos(v.size, q)
        out.append(v[lo] + t * (v[hi] - v[lo]))
    return np.asarray(out).astype(np.float32)


_orig_rtn = O.quantize_rtn


def _mut_rtn_scale_minus_one(w, b_max):
    w = np.asarray(w, np.float32)
    lo, hi = np.fmin.reduce(w, axis=1), np.fmax.reduce(w, axis=1)
    s = ((hi - lo) / np.float32((1 << b_max) - 1)).astype(np.float16)
    z = lo.astype(np.float16)
    with np.errstate(invalid="ignore", divide="ignore"):
        u = np.floor((w - z.astype(np.float32)[:, None]) / s.astype(np.float32)[:, None])
    u = np.clip(np.nan_to_num(u, nan=0.0), 0, (1 << b_max) - 1)
    return u.astype(np.uint8), s, z


def _mut_rtn_round_not_floor(w, b_max):
    q, s, z = _orig_rtn(w, b_max)
    w = np.asarray(w, np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        u = np.rint((w - z.astype(np.float32)[:, None]) / s.astype(np.float32)[:, None])
    u = np.clip(np.nan_to_num(u, nan=0.0), 0, (1 << b_max) - 1)
    return u.astype(np.uint8), s, z


def _mut_prefill_no_midpoint(X, q, s, z, b_max):
    X = np.asarray(X, np.float64)
    codes = (np.asarray(q, np.int64) & ((1 << b_max) - 1)).astype(np.float64)
    return X @ (np.asarray(s, np.float64)[:, None] * codes + np.asarray(z, np.float64)[:, None]).T


def _mut_prefill_scale_on_inputs(X, q, s, z, b_max):
    X = np.asarray(X, np.float64)
    codes = (np.asarray(q, np.int64) & ((1 << b_max) - 1)).astype(np.float64)
    s64, z64 = np.asarray(s, np.float64), np.asarray(z, np.float64)
    s_in = np.resize(s64, codes.shape[1])                 # s read along the input channels
    return X @ (s_in[None, :] * (codes + 0.5) + z64[:, None]).T


def _mut_prefill_top_planes_only(X, q, s, z, b_max):
    full = np.full(np.asarray(X).shape[-1], max(b_max - 2, 2), dtype=np.int64)
    w = O.dequant(O.truncated_codes(q, full, b_max), full, s, z, b_max)
    return np.asarray(X, np.float64) @ w


MUTATIONS = {
    "prefill_without_midpoint": ("prefill_gemm", _mut_prefill_no_midpoint),
    "prefill_scale_per_input_channel": ("prefill_gemm", _mut_prefill_scale_on_inputs),
    "prefill_drops_the_last_plane": ("prefill_gemm", _mut_prefill_top_planes_only),
    "rtn_scale_uses_levels_minus_one": ("quantize_rtn", _mut_rtn_scale_minus_one),
    "rtn_rounds_instead_of_floor": ("quantize_rtn", _mut_rtn_round_not_floor),
    "quantile_index_uses_n": ("quantile_position", _mut_quantile_index_n),
    "quantile_not_interpolated": ("quantile_position", _mut_quantile_no_interpolation),
    "calibration_on_signed_values": ("calibrate_thresholds", _mut_calibration_signed),
    "phi_exponent_off_by_one": ("phi", _mut_phi_exponent),
    "phi_zero_at_b_max": ("phi", _mut_phi_zero_at_full),
    "ties_go_down": ("assign_bits", _mut_ties_down),
    "planes_lsb_first": ("pack_planes", _mut_planes_lsb_first),
    "fragments_reversed_in_word": ("pack_planes", _mut_word_order_reversed),
    "z_dropped": ("dequant", _mut_drop_z),
    "rounding_instead_of_truncation": ("truncated_codes", _mut_round_not_truncate),
    "level_off_by_one": ("assign_bits", _mut_level_count_off_by_one),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch, golden_dir):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failures = 0
    for pin in _pins(golden_dir):
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures > 0, f"no pin caught mutation {name}"


def test_pins_pass_without_mutation(golden_dir):
    for pin in _pins(golden_dir):
        pin()
