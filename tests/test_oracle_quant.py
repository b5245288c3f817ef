"""Pins for the oracle's int8 quantisation on either side of W8A8: per-token
absmax quantisation of activations, and requantisation of int8 weights to
power-of-two scales ("Deterministic LLM Inference ... Power-of-Two INT8
Quantization Scales", section V).  Each check is a fact the definition fixes
(exact cases, invariances, bounds, hand-worked scales), not a restatement of
the oracle's code."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def f32(x):
    return np.float32(x)


# ---- activations, per token ---------------------------------------------------
def test_integer_rows_with_absmax_127_are_exact():
    """absmax 127 gives scale 127/127 = 1 exactly, so every integer maps to itself."""
    rng = np.random.default_rng(1)
    X = rng.integers(-127, 128, size=(8, 300)).astype(np.float32)
    X[:, 7] = 127.0
    X[3, 7] = -127.0
    Q, s = oracle.quantize_rows_int8(X)
    assert np.all(s == 1.0)
    assert np.array_equal(Q.astype(np.float32), X)


def test_zero_row_has_scale_one_and_zero_codes():
    X = np.zeros((3, 17), dtype=np.float32)
    X[1, 5] = 2.0
    Q, s = oracle.quantize_rows_int8(X)
    assert s[0] == 1.0 and s[2] == 1.0 and not Q[0].any() and not Q[2].any()
    assert Q[1, 5] == 127


def test_absmax_element_maps_to_full_scale_and_signs_mirror():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((64, 513)).astype(np.float32)
    Q, s = oracle.quantize_rows_int8(X)
    Qn, sn = oracle.quantize_rows_int8(-X)
    assert np.array_equal(s, sn) and np.array_equal(Qn, -Q)
    j = np.argmax(np.abs(X), axis=1)
    assert np.all(np.abs(Q[np.arange(64), j]) == 127)


def test_power_of_two_rescaling_is_invisible():
    """Multiplying a row by 2^j multiplies its scale by 2^j and leaves the
    codes alone (both the scale division and x / scale are exact in the
    exponent)."""
    rng = np.random.default_rng(3)
    X = rng.standard_normal((16, 200)).astype(np.float32)
    Q, s = oracle.quantize_rows_int8(X)
    for j in (-20, -3, 5, 30):
        Qj, sj = oracle.quantize_rows_int8(np.ldexp(X, j).astype(np.float32))
        assert np.array_equal(Qj, Q) and np.array_equal(sj, np.ldexp(s, j).astype(np.float32))


def test_exact_halves_round_to_even():
    """absmax 127/8 makes the scale exactly 1/8, so x = (k + 1/2) / 8 divides
    to an exact half and must go to the even neighbour."""
    k = np.arange(-126, 126)
    row = ((k + 0.5) / 8.0).astype(np.float32)
    X = np.concatenate([row, [np.float32(127 / 8)]])[None, :].astype(np.float32)
    Q, s = oracle.quantize_rows_int8(X)
    assert s[0] == np.float32(0.125)
    expect = np.where(k % 2 == 0, k, k + 1)  # k + 1/2 -> the even one of k, k+1
    assert np.array_equal(Q[0, :-1].astype(np.int64), expect)


def test_reconstruction_error_is_within_half_a_step():
    """|x - q s| <= s (1/2 + 127 u): the code is the nearest integer to a
    once-rounded quotient no larger than about 127 in size."""
    rng = np.random.default_rng(4)
    X = (rng.standard_normal((32, 1000)) * np.exp(rng.uniform(-10, 10, (32, 1)))).astype(np.float32)
    Q, s = oracle.quantize_rows_int8(X)
    err = np.abs(X.astype(np.float64) - Q.astype(np.float64) * s[:, None].astype(np.float64))
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -24))


def _rne_f32(fr):
    """A Fraction rounded to the nearest float32, ties to even (normal range)."""
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    if a == 0:
        return np.float32(0.0)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return np.float32(sign * float(q * ulp))


def test_against_exact_rational_evaluation():
    """Scale and codes evaluated with exact fractions and an independent
    round-to-nearest-even: fp32(amax/127), then rint(fp32(x/scale))."""
    rng = np.random.default_rng(5)
    X = rng.standard_normal((4, 64)).astype(np.float32)
    Q, s = oracle.quantize_rows_int8(X)
    for m in range(4):
        amax = max(abs(Fraction(float(v))) for v in X[m])
        sc = _rne_f32(amax / 127)
        assert s[m] == sc
        for k in range(64):
            t = Fraction(float(_rne_f32(Fraction(float(X[m, k])) / Fraction(float(sc)))))
            fl = t.numerator // t.denominator
            rem = t - fl
            code = fl + 1 if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2) else fl
            assert Q[m, k] == max(-127, min(127, code))


# ---- weights, to power-of-two scales ----------------------------------------
@pytest.mark.parametrize("s,nearest,ceil", [
    (0.75, 1.0, 1.0),          # log2 0.75 = -0.415: nearest 2^0
    (0.7, 0.5, 1.0),           # log2 0.7 = -0.515: nearest 2^-1
    (0.5, 0.5, 0.5),           # already a power of two
    (3.0, 4.0, 4.0),           # log2 3 = 1.585
    (2.8, 2.0, 4.0),           # log2 2.8 = 1.485
    (1.41421353816986083984375, 1.0, 2.0),   # the float just below sqrt 2
    (1.41421365737915039062500, 2.0, 2.0),   # the float just above sqrt 2
    (2.0 ** -30 * 1.5, 2.0 ** -29, 2.0 ** -29),
])
def test_hand_worked_power_of_two_scales(s, nearest, ceil):
    assert oracle.pow2_scale(s, "nearest") == nearest
    assert oracle.pow2_scale(s, "ceil") == ceil


def test_scale_bounds_and_mode_relation():
    rng = np.random.default_rng(6)
    s = np.exp(rng.uniform(-30, 10, 2000)).astype(np.float32)
    for v in s:
        n, c = oracle.pow2_scale(v, "nearest"), oracle.pow2_scale(v, "ceil")
        for p in (n, c):  # a power of two
            m, _ = np.frexp(p)
            assert m == 0.5
        v64 = float(v)
        assert v64 <= c < 2 * v64                       # ceiling never shrinks
        assert n * n * 2 >= v64 * v64 and n * n <= 2 * v64 * v64   # within sqrt 2 either way
        assert c in (n, 2 * n)


def test_power_of_two_scales_leave_weights_unchanged():
    rng = np.random.default_rng(7)
    W = rng.integers(-127, 128, (50, 96)).astype(np.int8)
    s = np.ldexp(np.ones(50), -rng.integers(1, 20, 50)).astype(np.float32)
    for mode in ("nearest", "ceil"):
        W2, s2 = oracle.requantize_pow2(W, s, mode)
        assert np.array_equal(W2, W) and np.array_equal(s2, s)


def test_requantised_weights_stay_within_half_a_new_step():
    """|q2 s2 - fp32(q s)| <= s2 / 2 unless the value clips at 127.5 s2; a
    second requantisation changes nothing (its scales are powers of two)."""
    rng = np.random.default_rng(8)
    W = rng.integers(-127, 128, (200, 64)).astype(np.int8)
    s = np.exp(rng.uniform(-12, -2, 200)).astype(np.float32)
    for mode in ("nearest", "ceil"):
        W2, s2 = oracle.requantize_pow2(W, s, mode)
        t = (W.astype(np.float32) * s[:, None]).astype(np.float64)
        back = W2.astype(np.float64) * s2[:, None].astype(np.float64)
        clipped = np.abs(t) > 127.5 * s2[:, None]
        assert np.all(np.abs(back - t)[~clipped] <= s2[:, None].repeat(64, 1)[~clipped] / 2)
        assert np.all(np.abs(W2[clipped]) == 127)
        if mode == "ceil":
            assert not clipped.any()      # a scale that never shrinks never clips
        W3, s3 = oracle.requantize_pow2(W2, s2, mode)
        assert np.array_equal(W3, W2) and np.array_equal(s3, s2)


def test_rows_without_a_usable_scale_are_copied():
    W = np.arange(-6, 6, dtype=np.int8).reshape(3, 4)
    s = np.array([0.0, -1.0, np.inf], dtype=np.float32)
    W2, s2 = oracle.requantize_pow2(W, s)
    assert np.array_equal(W2, W) and np.array_equal(s2, s, equal_nan=True)
