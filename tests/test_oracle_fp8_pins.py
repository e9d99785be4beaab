"""Pins of the FP8 oracle (``oracle/fp8.py``): Q and K multiplied by one random
orthogonal Hadamard matrix, quantised per row to E4M3, then the plain forward.

The pages (CMU 11-868 FlashAttention notes at quidproquo.cc, "FlashAttention-3:
asynchrony and FP8 on Hopper", slide page 24) fix the identity
(QJ)(KJ)^T = QK^T and that the rotation lowers the quantisation error on data
with outliers.  Checked here against things other than the oracle itself:
scipy's Hadamard matrix, orthogonality, the spreading of a single spike (closed
form), the E4M3 value set enumerated from its bit patterns, torch's float8_e4m3fn
cast, hand-rounded ties, the half-spacing error bound, a lossless construction
where the FP8 forward must equal the plain forward, and the outlier-error
reduction.  A dropped rotation on one side, a wrong sign pattern, a tie rounded
away from even, an off-by-one binade or a scale applied the wrong way fails one
of them.
"""
import math

import numpy as np
import pytest
import scipy.linalg
import torch

import oracle
from helpers import score_shift
from oracle import fp8

RNG = np.random.default_rng(20261204)


def signs(d):
    return RNG.choice([-1.0, 1.0], size=d)


def e4m3_values_from_bit_patterns():
    """Every non-negative finite E4M3 value, from the 7 magnitude bits of the
    byte: exponent field E (4 bits, bias 7), mantissa field f (3 bits); E = 0 is
    subnormal, and E = 15 with f = 7 is NaN."""
    vals, even = [], []
    for b in range(127):                     # 127 = 0b1111111 is NaN
        E, f = b >> 3, b & 7
        v = f * 2.0 ** -9 if E == 0 else (1 + f / 8) * 2.0 ** (E - 7)
        vals.append(v)
        even.append(f % 2 == 0)
    return np.array(vals), np.array(even)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128])
def test_sylvester_hadamard_matches_scipy(d):
    np.testing.assert_array_equal(fp8.sylvester_hadamard(d), scipy.linalg.hadamard(d))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_is_orthogonal_and_preserves_scores(d):
    J = fp8.rotation(signs(d))
    np.testing.assert_allclose(J @ J.T, np.eye(d), atol=1e-14)
    q, k = RNG.standard_normal((50, d)), RNG.standard_normal((70, d))
    np.testing.assert_allclose((q @ J) @ (k @ J).T, q @ k.T, atol=1e-11)


@pytest.mark.parametrize("d", [2, 16, 128])
def test_rotation_entries_closed_form(d):
    # Sylvester's matrix has H[i, j] = (-1)^popcount(i AND j); the random sign
    # s_i multiplies row i, i.e. input coordinate i is sign-flipped first.
    sg = signs(d)
    want = np.array([[sg[i] * (-1.0) ** bin(i & j).count("1") for j in range(d)]
                     for i in range(d)]) / math.sqrt(d)
    np.testing.assert_array_equal(fp8.rotation(sg), want)


def test_rotation_spreads_a_spike_evenly():
    d = 128
    x = np.zeros(d)
    x[37] = 10.0
    y = x @ fp8.rotation(signs(d))
    np.testing.assert_allclose(np.abs(y), np.full(d, 10.0 / math.sqrt(d)), rtol=1e-14)


def test_rotation_rejects_bad_input():
    with pytest.raises(ValueError):
        fp8.sylvester_hadamard(96)
    with pytest.raises(ValueError):
        fp8.rotation(np.array([1.0, 0.5]))


def test_e4m3_value_set_is_fixed_points():
    vals, _ = e4m3_values_from_bit_patterns()
    assert len(vals) == 127 and vals.max() == 448.0 and vals[1] == 2.0 ** -9
    np.testing.assert_array_equal(fp8.round_e4m3(vals), vals)
    np.testing.assert_array_equal(fp8.round_e4m3(-vals), -vals)


def test_e4m3_ties_go_to_the_even_mantissa():
    vals, even = e4m3_values_from_bit_patterns()
    mid = (vals[:-1] + vals[1:]) / 2         # exact in float64
    got = fp8.round_e4m3(mid)
    want = np.where(even[:-1], vals[:-1], vals[1:])
    np.testing.assert_array_equal(got, want)


def test_e4m3_hand_rounded_values():
    x = np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 0.0, -17.0, 19.0, 1.96875,
                  464.0, 470.0, -1e6])
    want = np.array([1.0, 1.25, 0.0, 2.0 ** -8, 0.0, -16.0, 20.0, 2.0, 448.0, 448.0, -448.0])
    np.testing.assert_array_equal(fp8.round_e4m3(x), want)


def test_e4m3_matches_torch_float8_cast():
    x = np.concatenate([RNG.uniform(-448, 448, 20000),
                        RNG.standard_normal(20000) * 2.0 ** RNG.integers(-12, 8, 20000)])
    x = np.clip(x, -448, 448)
    vals, _ = e4m3_values_from_bit_patterns()
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([x, mids, -mids])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(fp8.round_e4m3(x), ref)


def test_row_quantisation_error_is_within_half_a_spacing():
    x = RNG.standard_normal((40, 128)) * 2.0 ** RNG.integers(-20, 20, (40, 1))
    x[:, 5] *= 50                           # an outlier channel
    x[3] = 0.0                              # an all-zero row
    codes, scales = fp8.quantize_rows(x)
    assert scales[3] == 1.0 and not codes[3].any()
    np.testing.assert_array_equal(np.delete(np.abs(codes).max(axis=1), 3), 448.0)
    err = np.abs(codes * scales[:, None] - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None] * 2.0 ** -10)
    assert (err <= bound * (1 + 1e-12)).all()


def test_lossless_inputs_give_the_plain_forward():
    # Rows whose rotated values already lie on the E4M3 grid, with 448 as the
    # largest magnitude, quantise without loss (scale 1); for d = 64 every
    # product and sum below is exact in float64.
    d, n, scale = 64, 90, 0.125
    vals, _ = e4m3_values_from_bit_patterns()
    s = signs(d)
    J = fp8.rotation(s)

    def grid_rows(m):
        r = RNG.choice(vals[vals <= 8.0], size=(m, d)) * RNG.choice([-1.0, 1.0], size=(m, d))
        r[np.arange(m), RNG.integers(0, d, m)] = 448.0 * RNG.choice([-1.0, 1.0], size=m)
        return r

    qr, kr = grid_rows(n), grid_rows(n)
    q, k = qr @ J.T, kr @ J.T
    np.testing.assert_array_equal(q @ J, qr)
    np.testing.assert_array_equal(fp8.dequantized_rotated(q, s), qr)
    v = RNG.standard_normal((n, d))
    for causal in (False, True):
        o8, l8 = fp8.fp8_forward_head(q, k, v, causal, scale, s)
        o, lse = oracle.forward_head(q, k, v, causal, scale)
        np.testing.assert_allclose(o8, o, atol=1e-10)
        np.testing.assert_allclose(l8, lse, atol=1e-10)


def test_rotation_lowers_the_quantisation_error_with_outliers():
    # Simulated outliers: a few channels of Q and K 20x larger.  Quantised without
    # the rotation, each row's scale is set by its outlier and the other channels
    # lose most of their bits; with it, the error of the scores drops severalfold.
    n, d, scale = 256, 128, 1 / math.sqrt(128)
    q, k = RNG.standard_normal((n, d)), RNG.standard_normal((n, d))
    for c in (3, 40, 97):
        q[:, c] *= 20
        k[:, c] *= 20
    exact = scale * q @ k.T

    def deq(x):
        codes, sc = fp8.quantize_rows(x)
        return codes * sc[:, None]

    plain = np.linalg.norm(scale * deq(q) @ deq(k).T - exact) / np.linalg.norm(exact)
    rotated = np.linalg.norm(fp8.fp8_scores(q, k, signs(d), scale) - exact) / np.linalg.norm(exact)
    assert plain / rotated >= 2.0, (plain, rotated)


def test_fp8_forward_is_close_to_the_exact_forward():
    # Inputs from a generator of the test's own, so that they do not depend on
    # which tests ran before in the same process.  Since (QJ)(KJ)^T = QK^T, the
    # FP8 scores differ from the exact ones only by the rounding to E4M3; per
    # row, a score shift of at most delta moves LSE by at most delta and O by at
    # most (e^(2 delta) - 1) max|V|.  Over 200 seeds the relative O error stayed
    # below 0.04.
    rng = np.random.default_rng(11868)
    n, d, scale = 200, 128, 1 / math.sqrt(128)
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    s = rng.choice([-1.0, 1.0], size=d)
    qd, kd = fp8.dequantized_rotated(q, s), fp8.dequantized_rotated(k, s)
    for causal in (False, True):
        o8, l8 = fp8.fp8_forward_head(q, k, v, causal, scale, s)
        o, lse = oracle.forward_head(q, k, v, causal, scale)
        delta = score_shift(qd, kd, q, k, scale, causal)
        assert 0 < delta.max() < 0.5
        assert (np.abs(l8 - lse) <= delta + 1e-12).all()
        assert (np.abs(o8 - o) <= (np.expm1(2 * delta) * np.abs(v).max())[:, None] + 1e-12).all()
        assert np.linalg.norm(o8 - o) / np.linalg.norm(o) < 5e-2


@pytest.mark.parametrize("causal", [False, True])
def test_score_shift_bounds_used_by_the_fp8_forward_tolerance(causal):
    # The end-to-end FP8 parity test allows the GPU's codes to differ from the
    # oracle's (a rounding decision taken in fp32 instead of fp64): a per-row
    # shift of at most delta in the scores moves O by at most
    # (e^(2 delta) - 1) max|V| and LSE by at most delta.  Checked here on the
    # oracle with codes moved by one E4M3 step, and shown to be tight enough
    # that moving several codes per row does exceed a bound ten times smaller.
    n, d, scale = 96, 64, 0.125
    s = signs(d)
    q, k, v = (RNG.standard_normal((n, d)) for _ in range(3))
    J = fp8.rotation(s)
    qc, qs = fp8.quantize_rows(q @ J)
    kc, ks = fp8.quantize_rows(k @ J)
    o_ref, l_ref = oracle.forward_head(qc * qs[:, None], kc * ks[:, None], v, causal, scale)
    vals, _ = e4m3_values_from_bit_patterns()
    grid = np.concatenate([-vals[::-1], vals[1:]])
    shifted_any = False
    for trial in range(5):
        qc2, kc2 = qc.copy(), kc.copy()
        for c in (qc2, kc2):
            rows = RNG.integers(0, n, size=12)
            cols = RNG.integers(0, d, size=12)
            for r, col in zip(rows, cols):            # to a neighbouring E4M3 value
                i = np.searchsorted(grid, c[r, col])
                c[r, col] = grid[min(len(grid) - 1, i + 1)] if RNG.random() < 0.5 else grid[max(0, i - 1)]
        a_q, a_k = qc2 * qs[:, None], kc2 * ks[:, None]
        o2, l2 = oracle.forward_head(a_q, a_k, v, causal, scale)
        delta = score_shift(a_q, a_k, qc * qs[:, None], kc * ks[:, None], scale, causal)
        bound_o = np.expm1(2 * delta)[:, None] * np.abs(v).max()
        assert (np.abs(o2 - o_ref) <= bound_o + 1e-12).all()
        assert (np.abs(l2 - l_ref) <= delta + 1e-12).all()
        shifted_any |= bool((np.abs(l2 - l_ref) > delta / 10).any())
    assert shifted_any
