"""Pins that hold the CPU oracle to the GRINQH note and to mathematics.

No pin retypes the oracle's own formulas: each compares it with something
else - values derived by hand from the page (tests/golden), a library
routine the special case reduces to, a closed form, an invariant, or a brute
force that reaches the same number by a different mechanism (bit strings,
enumeration of truncation intervals).

"KD1/KD2/KD3" are items 1-3 of the key-design section (方法详解 / 关键设计) of
"GRINQH: Graded Input-Based Quantization Hierarchy for Efficient LLM
Generation" (papernotes.org note).
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import grinqh_oracle as O
from oracle import c_oracle as C
import synthetic as S


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- KD1 -------

def test_assign_bits_golden_ties(golden_dir):
    g = _load(golden_dir, "assign_bits_ties.json")
    x = np.array([float(v) for v in g["x"]], dtype=np.float32)
    bits = O.assign_bits(x, np.array(g["theta"], np.float32), g["b_max"])
    assert bits.tolist() == g["bits"]
    assert C.assign_bits(x, np.array(g["theta"], np.float32), g["b_max"]).tolist() == g["bits"]


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_assign_bits_is_searchsorted(b_max):
    """For finite x and ascending thresholds, the level is numpy's right-side
    insertion index of |x| into the thresholds (interval [theta_k, theta_k+1))."""
    rng = np.random.default_rng(7 + b_max)
    P = b_max // 2
    theta = np.sort(rng.uniform(0.0, 3.0, P)).astype(np.float32)
    x = rng.standard_normal(20000).astype(np.float32) * 2
    # exact ties, one ulp either side, signed zeros
    ties = np.concatenate([theta, -theta, np.nextafter(theta, np.float32(0)),
                           np.nextafter(theta, np.float32(np.inf)), [0.0, -0.0]]).astype(np.float32)
    x = np.concatenate([x, ties])
    expect = 2 * np.searchsorted(theta.astype(np.float64), np.abs(x.astype(np.float64)), side="right")
    assert np.array_equal(O.assign_bits(x, theta, b_max), expect.astype(np.uint8))
    assert np.array_equal(C.assign_bits(x, theta, b_max), expect.astype(np.uint8))


def test_assign_bits_special_values():
    theta = np.array([0.0, 0.0, 1.0, 1.0], np.float32)   # equal thresholds: empty levels
    x = np.array([0.0, -0.0, 0.5, 1.0, np.nan, np.inf], np.float32)
    # |x| >= 0 always (level 2 at least), NaN compares false everywhere
    assert O.assign_bits(x, theta, 8).tolist() == [4, 4, 4, 8, 0, 8]
    assert O.active_channels(O.assign_bits(x, theta, 8)).tolist() == [0, 1, 2, 3, 5]


# ---------------------------------------------------------------- KD2 -------

def test_pack_golden_hand_examples(golden_dir):
    g = _load(golden_dir, "pack_hand_example.json")
    for case in g["cases"]:
        q = np.array(case["q_out_by_in"], dtype=np.uint8)
        expect = np.array(case["planes"], dtype=np.uint32)
        assert np.array_equal(O.pack_planes(q, case["b_max"]), expect)
        assert np.array_equal(C.pack_planes(q, case["b_max"]), expect)


@pytest.mark.parametrize("b_max,d_in,d_out", [(8, 5, 1), (8, 3, 130), (4, 7, 64), (6, 2, 65), (2, 9, 200)])
def test_pack_round_trip(b_max, d_in, d_out):
    rng = np.random.default_rng(b_max * 1000 + d_out)
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    q[0, 0] = 0
    q[-1, -1] = (1 << b_max) - 1
    planes = O.pack_planes(q, b_max)
    assert planes.shape == (d_in, b_max // 2, O.row_words(d_out))
    frag = O.unpack_fragments(planes, d_out).astype(np.int64)
    P = b_max // 2
    rebuilt = sum(frag[:, p, :] << (b_max - 2 * p - 2) for p in range(P))
    assert np.array_equal(rebuilt, q.T.astype(np.int64))
    # padding fragments are zero
    full = ((planes[:, :, :, None] >> (2 * np.arange(16, dtype=np.uint32))) & 3).reshape(d_in, P, -1)
    assert not full[:, :, d_out:].any()
    assert np.array_equal(C.pack_planes(q, b_max), planes)


# ---------------------------------------------------------------- KD3 -------

def _string_truncate(q, b, b_max):
    """Top b bits of q by string slicing, then zero-filled: a different mechanism."""
    s = format(int(q), f"0{b_max}b")
    return int(s[:b] + "0" * (b_max - b), 2) if b else 0


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_codes_exhaustive(b_max):
    """Every code q and every width b: the sum of the taken planes equals the
    zero-filled top-b-bit string of q (KD3's spliced truncated integer)."""
    q = np.arange(1 << b_max, dtype=np.uint8)[:, None]          # d_out = 2^b_max, d_in = 1
    planes = O.pack_planes(q, b_max)
    for b in range(2, b_max + 1, 2):
        bits = np.array([b])
        from_planes = O.codes_from_planes(planes, bits, b_max, q.shape[0])[0]
        direct = O.truncated_codes(q, bits, b_max)[0]
        expect = [_string_truncate(v, b, b_max) for v in range(1 << b_max)]
        assert from_planes.tolist() == expect
        assert direct.tolist() == expect


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_midpoint_is_interval_centroid(b_max):
    """w_hat_b(q) equals the mean of the full-width reconstructions s*(r + 1/2) + z
    over every code r that shares q's top b bits (brute-force enumeration), i.e.
    phi puts the point in the middle of the truncation interval (KD3)."""
    s, z = 0.0068359375, -0.0031280517578125      # fp16-exact values
    for b in range(2, b_max + 1, 2):
        k = b_max - b
        bits = np.array([b])
        for qv in range(1 << b_max):
            code = O.truncated_codes(np.array([[qv]], np.uint8), bits, b_max)[0, 0]
            w = O.dequant(np.array([[code]]), bits, [s], [z], b_max)[0, 0]
            top = qv >> k
            members = [r for r in range(1 << b_max) if (r >> k) == top]
            assert len(members) == 1 << k
            centroid = np.mean([s * (r + 0.5) + z for r in members])
            assert w == pytest.approx(centroid, rel=0, abs=1e-15)


def test_bias_table_closed_forms(golden_dir):
    g = _load(golden_dir, "bias_closed_forms.json")
    for b_max_s, table in g["tables"].items():
        got = O.bias_table(int(b_max_s))
        for b_s, row in table.items():
            for key, val in row.items():
                assert got[int(b_s)][key] == pytest.approx(val, abs=1e-12), (b_max_s, b_s, key)


# ------------------------------------------------------------- GEMV ---------

def test_tiny_gemv_golden(golden_dir):
    g = _load(golden_dir, "tiny_gemv_b4.json")
    q = np.array(g["q_out_by_in"], np.uint8)
    x = np.array(g["x"], np.float32)
    th = np.array(g["theta"], np.float32)
    bits = O.assign_bits(x, th, g["b_max"])
    assert bits.tolist() == g["bits"]
    codes = O.truncated_codes(q, bits, g["b_max"])
    assert codes.tolist() == g["codes_in_by_out"]
    w = O.dequant(codes, bits, g["s"], g["z"], g["b_max"])
    assert np.allclose(w, g["w_hat_in_by_out"], rtol=0, atol=1e-15)
    for y in (O.gemv(x, th, q, g["s"], g["z"], g["b_max"]),
              O.gemv(x, th, q, g["s"], g["z"], g["b_max"], exact=True),
              O.gemv_from_planes(x, th, O.pack_planes(q, g["b_max"]), g["s"], g["z"], g["b_max"], 2),
              C.gemv(x, th, q, g["s"], g["z"], g["b_max"])):
        assert np.allclose(y, g["y"], rtol=0, atol=1e-15)
    assert O.eff_bits(bits) == g["eff_bits"]


def _rand_problem(d_in, d_out, b_max, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 1 << b_max, size=(d_out, d_in), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d_out).astype(np.float16)
    z = rng.normal(0, 0.01, d_out).astype(np.float16)
    x = (rng.standard_t(3, d_in)).astype(np.float32)
    theta = np.sort(np.quantile(np.abs(x), np.linspace(0.2, 0.9, b_max // 2))).astype(np.float32)
    return q, s, z, x, theta


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_dense_mode_is_plain_dot(b_max):
    """All thresholds 0 -> every channel gets b_max bits; the product is numpy's
    dot of x with s_j*(q_ji + 1/2) + z_j built from q directly, never packed."""
    q, s, z, x, _ = _rand_problem(300, 70, b_max, 11)
    theta = np.zeros(b_max // 2, np.float32)
    W = s.astype(np.float64)[None, :] * (q.T.astype(np.float64) + 0.5) + z.astype(np.float64)[None, :]
    ref = np.dot(x.astype(np.float64), W)
    y = O.gemv(x, theta, q, s, z, b_max)
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))
    yc = C.gemv(x, theta, q, s, z, b_max)
    assert np.max(np.abs(yc - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_all_skipped_gives_exact_zero():
    q, s, z, x, _ = _rand_problem(200, 64, 8, 12)
    for theta in (np.full(4, np.inf, np.float32), np.full(4, 1e30, np.float32)):
        bits = O.assign_bits(x, theta, 8)
        assert O.active_channels(bits).size == 0
        assert np.all(O.gemv(x, theta, q, s, z, 8) == 0.0)
        assert np.all(C.gemv(x, theta, q, s, z, 8) == 0.0)
        assert O.required_bytes(bits, 64)["planes"] == 0.0


def test_single_active_channel():
    q, s, z, x, _ = _rand_problem(50, 64, 8, 13)
    x[:] = 0.01
    x[17] = -3.0
    theta = np.array([1.0, 2.0, 2.5, 9.0], np.float32)    # only |x_17| = 3 passes, 6 bits
    y = O.gemv(x, theta, q, s, z, 8)
    # 6 bits: k = 2, code = top six bits, midpoint offset = 2
    row = [float(s[j]) * (((int(q[j, 17]) >> 2) << 2) + 2.0) + float(z[j]) for j in range(64)]
    assert np.allclose(y, -3.0 * np.array(row, np.float64), rtol=1e-15, atol=0)


def test_bruteforce_8x8_all_level_patterns():
    """All 5^8 assignments of the 8 channels to the 5 levels of b_max = 8.
    Reference: per channel and level, the reconstructed row is the centroid of
    the full-width reconstructions over the truncation interval (enumerated),
    and y sums x_i times that row over channels with a non-zero level."""
    b_max, d = 8, 8
    rng = np.random.default_rng(88)
    q = rng.integers(0, 256, size=(d, d), dtype=np.uint8)
    s = rng.uniform(0.001, 0.01, d).astype(np.float16).astype(np.float64)
    z = rng.normal(0, 0.01, d).astype(np.float16).astype(np.float64)
    theta = np.array([0.5, 1.0, 2.0, 4.0], np.float32)
    mid = np.array([0.25, 0.75, 1.5, 3.0, 6.0])               # one magnitude inside each level
    # R[i, L, j]: reconstructed weight of channel i at level L (0 -> none)
    R = np.zeros((d, 5, d))
    for i in range(d):
        for L in range(1, 5):
            k = b_max - 2 * L
            for j in range(d):
                top = int(q[j, i]) >> k
                members = [r for r in range(256) if (r >> k) == top]
                R[i, L, j] = np.mean([s[j] * (r + 0.5) + z[j] for r in members])
    levels = np.array(list(itertools.product(range(5), repeat=d)), dtype=np.int64)   # [5^8][8]
    signs = np.where(rng.random(levels.shape) < 0.5, -1.0, 1.0)
    X = (signs * mid[levels]).astype(np.float32)
    ref = np.einsum("ni,nij->nj", X.astype(np.float64), R[np.arange(d)[None, :], levels, :])
    for lo in range(0, levels.shape[0], 65536):
        sl = slice(lo, lo + 65536)
        bits = O.assign_bits(X[sl], theta, b_max)
        assert np.array_equal(bits.astype(np.int64), 2 * levels[sl])
        y = O.gemv(X[sl], theta, q, s, z, b_max)
        assert np.max(np.abs(y - ref[sl])) <= 1e-12
    # the plane path and the C oracle on a sample of the patterns
    planes = O.pack_planes(q, b_max)
    for n in rng.choice(levels.shape[0], 300, replace=False):
        yp = O.gemv_from_planes(X[n], theta, planes, s, z, b_max, d)
        yc = C.gemv(X[n], theta, q, s, z, b_max)
        assert np.max(np.abs(yp - ref[n])) <= 1e-12
        assert np.max(np.abs(yc - ref[n])) <= 1e-12


def test_power_of_two_scale_invariance_and_permutation():
    q, s, z, x, theta = _rand_problem(513, 130, 8, 14)
    y = O.gemv(x, theta, q, s, z, 8)
    for m in (-3, 5):
        xs = np.ldexp(x, m).astype(np.float32)
        ts = np.ldexp(theta, m).astype(np.float32)
        assert np.array_equal(O.assign_bits(xs, ts, 8), O.assign_bits(x, theta, 8))
        assert np.array_equal(O.gemv(xs, ts, q, s, z, 8), np.ldexp(y, m))
    perm = np.random.default_rng(3).permutation(513)
    yp = O.gemv(x[perm], theta, q[:, perm], s, z, 8)
    assert np.max(np.abs(yp - y)) <= 1e-12 * np.max(np.abs(y))


@pytest.mark.parametrize("b_max", [4, 8])
def test_factorised_form(b_max):
    """y_j = s_j*(A_j + C) + z_j*S with A from the raw plane fragments weighted by
    x_i*4^(P-1-p), C = sum x_i*phi_i and S = sum x_i over loaded channels: the
    algebra a kernel can use, equal to the oracle's plain sum to 1e-12."""
    q, s, z, x, theta = _rand_problem(700, 200, b_max, 15)
    P = b_max // 2
    bits = O.assign_bits(x, theta, b_max)
    frag = O.unpack_fragments(O.pack_planes(q, b_max), 200).astype(np.float64)
    xd = x.astype(np.float64)
    A = np.zeros(200)
    Cs = 0.0
    Ss = 0.0
    for i in range(700):
        Pi = int(bits[i]) // 2
        if Pi == 0:
            continue
        for p in range(Pi):
            A += xd[i] * 4.0 ** (P - 1 - p) * frag[i, p]
        Cs += xd[i] * 2.0 ** (b_max - int(bits[i]) - 1)
        Ss += xd[i]
    yf = s.astype(np.float64) * (A + Cs) + z.astype(np.float64) * Ss
    y = O.gemv(x, theta, q, s, z, b_max)
    assert np.max(np.abs(yf - y)) <= 1e-12 * np.max(np.abs(y))


def test_required_bytes_counts_taken_plane_rows():
    q, s, z, x, theta = _rand_problem(999, 192, 8, 16)
    bits = O.assign_bits(x, theta, 8)
    rows = int(np.sum(bits // 2))
    rb = O.required_bytes(bits, 192)
    assert rb["planes"] == rows * O.row_words(192) * 4
    assert rb["total"] == rb["planes"] + 4 * 192


def test_nan_is_skipped_and_inf_propagates():
    q, s, z, x, theta = _rand_problem(64, 64, 8, 17)
    assert theta[0] > 0
    x_nan = x.copy()
    x_nan[5] = np.nan
    x_off = x.copy()
    x_off[5] = 0.0                       # below theta_1: not loaded
    assert O.assign_bits(x_nan, theta, 8)[5] == 0
    y_nan = O.gemv(x_nan, theta, q, s, z, 8)
    assert np.all(np.isfinite(y_nan))
    assert np.array_equal(y_nan, O.gemv(x_off, theta, q, s, z, 8))
    x_inf = x.copy()
    x_inf[3] = np.inf
    assert O.assign_bits(x_inf, theta, 8)[3] == 8
    assert not np.all(np.isfinite(O.gemv(x_inf, theta, q, s, z, 8)))


def test_c_oracle_matches_numpy_on_small_workload():
    L = S.make_linear(S.small_case())
    y = O.gemv(L.x, L.theta, L.q, L.s, L.z, 8)
    yc = C.gemv(L.x, L.theta, L.q, L.s, L.z, 8)
    assert np.max(np.abs(y - yc)) <= 1e-12 * np.max(np.abs(y))
    assert np.array_equal(O.pack_planes(L.q, 8), C.pack_planes(L.q, 8))


def test_synthetic_thresholds_hit_target_bits():
    L = S.make_linear(S.small_case())
    assert abs(O.eff_bits(O.assign_bits(L.x, L.theta, 8)) - 3.1) < 0.25
    for eff in (2, 3, 4):
        spec = S.llama8b_linears(eff)[0]
        Lx = S.make_linear(spec, with_codes=False)
        assert abs(O.eff_bits(O.assign_bits(Lx.x, Lx.theta, 8)) - eff) < 0.2
    Ld = S.make_linear(S.llama8b_linears(8)[0], with_codes=False)
    assert O.eff_bits(O.assign_bits(Ld.x, Ld.theta, 8)) == 8.0
    for eff in (2, 3, 4):
        spec = S.llama8b_linears_b6(eff)[0]
        Lx = S.make_linear(spec, with_codes=False)
        assert abs(O.eff_bits(O.assign_bits(Lx.x, Lx.theta, 6)) - eff) < 0.2
    L6 = S.make_linear(S.llama8b_linears_b6(6)[0], with_codes=False)
    assert O.eff_bits(O.assign_bits(L6.x, L6.theta, 6)) == 6.0


@pytest.mark.parametrize("table,b_max", [(S.QUANTILES_B8, 8), (S.QUANTILES_B6, 6), (S.QUANTILES_B4, 4)])
def test_quantile_tables_give_their_expected_bits(table, b_max):
    """Each table's cumulative levels imply level shares whose mean bit width
    is exactly the table key (None: every channel at b_max)."""
    for eff, q in table.items():
        if q is None:
            assert eff == b_max
            continue
        assert len(q) == b_max // 2 and all(a < b for a, b in zip(q, q[1:]))
        c = (0.0,) + tuple(q) + (1.0,)
        shares = [c[i + 1] - c[i] for i in range(len(c) - 1)]
        assert abs(sum(2 * i * sh for i, sh in enumerate(shares)) - eff) < 1e-12


def test_max_rel_error_metric():
    ref = np.array([1.0, -2.0, 0.0, 1e-9])
    assert O.max_rel_error(ref, ref) == 0.0
    rms = np.sqrt(np.mean(ref ** 2))
    y = ref + np.array([0, 0, 1e-3 * rms, 0])
    assert O.max_rel_error(y, ref) == pytest.approx(0.1, rel=1e-9)


def test_round_to_bf16_against_bit_arithmetic():
    """RNE to bf16 checked on hand-picked halfway cases and against numpy's own
    fp32 -> fp16-free route: exact values with <= 8 significant bits round-trip."""
    vals = np.array([1.0, 1.00390625, 1.01171875, -3.0, 0.0], np.float32)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    got = O.round_to_bf16(vals)
    back = (got.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0, 1.015625, -3.0, 0.0]


# ---------------------------------------------------- threshold calibration --

@pytest.mark.parametrize("n", [1, 2, 3, 1000, 4096 * 3 + 7])
def test_calibration_matches_numpy_linear_quantile(n):
    """The calibration quantile is numpy's linear method (numpy.quantile), up
    to one fp32 step where numpy interpolates from the upper value."""
    rng = np.random.default_rng(n)
    x = rng.standard_t(3, n).astype(np.float32)
    levels = [0.0, 0.2, 0.5, 0.73, 0.9999, 1.0]
    got = O.calibrate_thresholds(x, levels)
    ref = np.quantile(np.abs(x).astype(np.float64), levels).astype(np.float32)
    assert np.all(np.abs(got.view(np.int32).astype(np.int64) - ref.view(np.int32).astype(np.int64)) <= 1)
    assert np.mean(got == ref) >= 0.8


def test_calibration_closed_forms():
    # integer ramp 0..n-1: the quantile at q is (n - 1) q exactly (dyadic q)
    n = 1025
    v = np.arange(n, dtype=np.float32)
    for q in (0.0, 0.25, 0.5, 0.625, 1.0):
        assert O.calibrate_thresholds(v, [q])[0] == np.float32((n - 1) * q)
    # two values: a + q (b - a)
    assert O.calibrate_thresholds(np.array([2.0, -6.0], np.float32), [0.25])[0] == np.float32(3.0)
    # constant data, signs and order do not matter
    c = np.full(77, -1.5, np.float32)
    assert np.all(O.calibrate_thresholds(c, [0.0, 0.3, 1.0]) == np.float32(1.5))
    rng = np.random.default_rng(5)
    x = rng.normal(size=500).astype(np.float32)
    lv = [0.1, 0.5, 0.9]
    assert np.array_equal(O.calibrate_thresholds(x, lv), O.calibrate_thresholds(-x[::-1], lv))
    # the ends are the smallest and largest magnitudes
    assert O.calibrate_thresholds(x, [0.0])[0] == np.min(np.abs(x))
    assert O.calibrate_thresholds(x, [1.0])[0] == np.max(np.abs(x))


def test_calibration_ties_and_nan_order():
    # repeated values: any level inside a run of equal values returns that value
    v = np.array([1, 1, 1, 1, 4, 4, 4, 4], np.float32)
    assert O.calibrate_thresholds(v, [0.2, 0.4])[0] == 1.0
    assert O.calibrate_thresholds(v, [0.8])[0] == 4.0
    # NaN sorts after +Inf: low levels stay finite, the top level is NaN
    w = np.array([np.nan, 1.0, 2.0, np.inf], np.float32)
    got = O.calibrate_thresholds(w, [0.0, 0.5, 1.0])
    assert got[0] == 1.0 and np.isinf(got[1]) and np.isnan(got[2])
    # a level that lands on a value returns it, also next to +Inf
    assert O.calibrate_thresholds(np.array([1.0, 2.0, np.inf], np.float32), [0.5])[0] == 2.0
    assert O.calibrate_thresholds(np.array([1.0, np.inf], np.float32), [1.0])[0] == np.inf


def test_harness_thresholds_are_the_calibration_quantiles():
    """The synthetic harness's thresholds (numpy.quantile) agree with the
    calibration definition to within one fp32 step."""
    spec = S.llama8b_linears(3)[0]
    xs, _ = S.gen_x_stream(spec)
    calib = S.bf16_bits_to_f32(S.f32_to_bf16_bits(xs[:spec.n_calib]))
    th_h = S.calibrate_theta(calib, S.QUANTILES_B8[3], 4)
    th_o = O.calibrate_thresholds(calib, S.QUANTILES_B8[3])
    assert np.all(np.abs(th_h.view(np.int32).astype(np.int64) - th_o.view(np.int32).astype(np.int64)) <= 1)


# ------------------------------------------------------------ RTN front end --

@pytest.mark.parametrize("k", [0, 3, 9])
def test_rtn_codes_on_an_exact_integer_grid(k):
    """b_max 8: rows of grid points w = q * 2^-k (exact in bf16) with a 0 and a
    256 * 2^-k anchor have s = 2^-k, z = 0, and return their own q; the top
    anchor is clamped to 255."""
    rng = np.random.default_rng(k)
    q_true = rng.integers(0, 256, size=(6, 300))
    w = (q_true * 2.0 ** -k).astype(np.float32)
    w[:, 0] = 0.0
    w[:, 1] = 256 * 2.0 ** -k
    q_true[:, 0] = 0
    q_true[:, 1] = 255
    q, s, z = O.quantize_rtn(w, 8)
    assert np.all(s == np.float16(2.0 ** -k)) and np.all(z == 0)
    assert np.array_equal(q, q_true.astype(np.uint8))


def test_rtn_codes_at_interval_centres():
    """b_max 4: rows of interval centres w = (q + 1/2) * 2^-3 with 0 and 2 as
    anchors return q (a centre is never rounded up)."""
    rng = np.random.default_rng(4)
    q_true = rng.integers(0, 16, size=(5, 200))
    w = ((q_true + 0.5) * 0.125).astype(np.float32)
    w[:, 0], w[:, 1] = 0.0, 2.0
    q_true[:, 0], q_true[:, 1] = 0, 15
    q, s, z = O.quantize_rtn(w, 4)
    assert np.all(s == np.float16(0.125)) and np.all(z == 0)
    assert np.array_equal(q, q_true.astype(np.uint8))


@pytest.mark.parametrize("b_max", [2, 4, 6, 8])
def test_rtn_round_trip_bound(b_max):
    """Every weight is within half an interval of its midpoint reconstruction,
    up to the fp16 rounding of the stored scale and zero point."""
    rng = np.random.default_rng(b_max)
    w = rng.normal(0, 0.02, size=(64, 777)).astype(np.float32)
    w[::7, 5] *= 40.0                                    # outliers
    w = S.bf16_bits_to_f32(S.f32_to_bf16_bits(w))
    q, s, z = O.quantize_rtn(w, b_max)
    s64, z64 = s.astype(np.float64)[:, None], z.astype(np.float64)[:, None]
    w_hat = s64 * (q.astype(np.float64) + 0.5) + z64
    lo, hi = w.min(axis=1).astype(np.float64)[:, None], w.max(axis=1).astype(np.float64)[:, None]
    s_exact = (hi - lo) / 2.0 ** b_max
    bound = 0.5 * s64 + np.abs(z64 - lo) + 2.0 ** b_max * np.abs(s_exact - s64) + 1e-12
    assert np.all(np.abs(w_hat - w) <= bound)
    # and mostly within the half interval itself
    assert np.mean(np.abs(w_hat - w) <= 0.5 * s64 * (1 + 1e-6)) > 0.98
    # codes never decrease as the weight grows
    for j in range(0, 64, 9):
        o = np.argsort(w[j], kind="stable")
        assert np.all(np.diff(q[j][o].astype(np.int64)) >= 0)


def test_rtn_special_rows():
    w = np.array([[1.5] * 8,                                           # constant
                  [np.nan, 1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0],        # NaN ignored in min / max
                  [0.0, 1.0, np.inf, 2.0, 3.0, 4.0, 5.0, 6.0]], np.float32)
    q, s, z = O.quantize_rtn(w, 4)
    assert s[0] == 0 and z[0] == np.float16(1.5) and np.all(q[0] == 0)
    assert z[1] == 1.0 and s[1] == np.float16(6.0 / 16) and q[1, 0] == 0
    assert q[1, 7] == 15 and q[1, 1] == 0
    assert np.isinf(s[2]) and np.all(q[2] == 0)


# ------------------------------------------------------------- prefill ------

def test_prefill_integer_exact():
    """s = 1, z = 0 and integer X: 2Y is the exact integer product X (2Q + 1)^T,
    which fixes the midpoint at b_max and the orientation of Q (non-square)."""
    rng = np.random.default_rng(21)
    for b_max in (2, 4, 6, 8):
        M, d_in, d_out = 5, 7, 11
        q = rng.integers(0, 256, size=(d_out, d_in))           # high bits are not part of the code
        X = rng.integers(-9, 10, size=(M, d_in))
        Y = O.prefill_gemm(X.astype(np.float64), q.astype(np.uint8), np.ones(d_out), np.zeros(d_out), b_max)
        codes = q & ((1 << b_max) - 1)
        assert np.array_equal(2 * Y, (X @ (2 * codes + 1).T).astype(np.float64))


def test_prefill_constant_codes_closed_form():
    """q = c, s = sigma, z = zeta everywhere: every weight is sigma (c + 1/2) + zeta,
    so Y[m][j] is that times the row sum of X."""
    rng = np.random.default_rng(22)
    X = rng.normal(size=(4, 33))
    for b_max, c in ((8, 200), (4, 9), (2, 3), (6, 0)):
        sigma, zeta = 0.375, -0.0625
        q = np.full((19, 33), c, np.uint8)
        Y = O.prefill_gemm(X, q, np.full(19, sigma), np.full(19, zeta), b_max)
        w = sigma * (c + 0.5) + zeta
        assert np.allclose(Y, w * X.sum(axis=1)[:, None], rtol=1e-13, atol=1e-13)


def test_prefill_of_rtn_weights_approximates_the_weights():
    """RTN onto the b_max midpoint grid, then the prefill product: each output is
    within sum_i |X_mi| * (half an interval, plus the fp16 rounding of s and z)
    of X W^T.  Square and per-output scales, so s or z taken along the wrong
    axis breaks the bound."""
    rng = np.random.default_rng(23)
    n = 96
    w = rng.normal(0, 0.02, size=(n, n)).astype(np.float32)
    w *= rng.uniform(0.2, 5.0, size=(n, 1)).astype(np.float32)      # rows of very different range
    X = rng.normal(size=(6, n))
    for b_max in (4, 8):
        q, s, z = O.quantize_rtn(w, b_max)
        Y = O.prefill_gemm(X, q, s, z, b_max)
        s64, z64 = s.astype(np.float64), z.astype(np.float64)
        lo = w.min(axis=1).astype(np.float64)
        per_w = 0.5 * s64 + np.abs(z64 - lo) + 2.0 ** b_max * np.abs((w.max(axis=1) - lo) / 2.0 ** b_max - s64)
        bound = np.abs(X) @ np.broadcast_to(per_w, (n, n)) + 1e-12
        assert np.all(np.abs(Y - X @ w.astype(np.float64).T) <= bound)
