"""Pins for the oracle's scalar primitives against library routines and the
IEEE-754 definition (exact rationals)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import f32_value, round_f32, round_float

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_bf16_rne_matches_torch_cast():
    """fp32 -> bf16 round-to-nearest-even against torch's CPU cast (a library
    routine), over every upper half-word with the lower half-words that decide
    the rounding (0, just below / at / above the halfway point, all ones) and
    random ones."""
    import torch
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    rng = np.random.default_rng(7)
    lows = np.concatenate([np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32),
                           rng.integers(0, 1 << 16, size=26).astype(np.uint32)])
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    x = u.view(np.float32)
    got = oracle.bf16_rne(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])
    # NaN stays NaN (quiet, sign kept)
    g = got[nan]
    assert np.all((g & 0x7F80) == 0x7F80) and np.all(g & 0x7F)
    assert np.array_equal(g >> 15, (u[nan] >> 31).astype(np.uint16))


def test_bf16_rne_ties_to_even_by_definition():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to the even significand 1
    assert oracle.bf16_rne(np.float32(1 + 2 ** -8))[()] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1+2^-7 (odd) and 1+2^-6 (even)
    assert oracle.bf16_rne(np.float32(1 + 3 * 2 ** -8))[()] == 0x3F82
    # past the halfway point above the largest finite bf16 rounds to inf;
    # exactly halfway goes to the even neighbour, which is inf as well
    over = np.array([0x7F7F8001, 0x7F7F8000, 0x7F7F7FFF], dtype=np.uint32).view(np.float32)
    assert list(oracle.bf16_rne(over)) == [0x7F80, 0x7F80, 0x7F7F]


def test_int_to_f32_rne_matches_numpy():
    rng = np.random.default_rng(3)
    v = np.concatenate([np.arange(-70000, 70000), rng.integers(-(1 << 25), 1 << 25, 20000),
                        np.array([2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 24 + 1), 2 ** 31 - 1, -(2 ** 31)])])
    for x in v[::7]:
        assert oracle.f32_from_i32(int(x)) == np.float32(np.int64(x).astype(np.float32))
    # and against the definition, around 2^24 where rounding starts
    for x in range(2 ** 24 - 8, 2 ** 24 + 40):
        assert oracle.f32_from_i32(x) == round_f32(Fraction(x))


@pytest.mark.parametrize("mode", ["rne", "rz"])
def test_round_sum_is_correct_rounding_of_exact_sum(mode):
    """The wide accumulator's one rounding equals the IEEE definition applied
    to the exact rational sum, on ordinary, cancelling, subnormal and
    overflowing sums."""
    rng = np.random.default_rng(11)
    for trial in range(3000):
        n = int(rng.integers(1, 12))
        terms = []
        for _ in range(n):
            s = int(rng.integers(0, 2))
            mag = int(rng.integers(0, 1 << int(rng.integers(1, 40))))
            e = int(rng.integers(-250, 100)) if trial % 3 else int(rng.integers(-180, -120))
            terms.append((s, mag, e))
        if trial % 5 == 0:  # exact cancellation of the top term
            s, mag, e = terms[0]
            terms.append((1 - s, mag, e))
        exact = sum((-1 if s else 1) * Fraction(m) * Fraction(2) ** e for s, m, e in terms)
        got = oracle.round_sum(terms, mode)
        ref = round_float(exact, 24, -126, 127, mode)
        if isinstance(ref, float):  # inf
            assert got == ref
        else:
            assert Fraction(float(got)) == ref, (terms, got, ref)


def test_round_sum_overflow_and_signed_zero():
    big = (0, (1 << 24) - 1, 104)  # fp32 max
    half_ulp = (0, 1, 103)
    assert oracle.round_sum([big, half_ulp], "rne") == np.inf
    assert oracle.round_sum([big, half_ulp], "rz") == np.float32(3.4028235e38)
    z = oracle.round_sum([(1, 0, 0), (1, 0, 5)])
    assert z == 0 and np.signbit(z)
    z = oracle.round_sum([(0, 3, 0), (1, 3, 0)])
    assert z == 0 and not np.signbit(z)


def test_fmaf_single_rounding_via_sumsq_leaf():
    """A one-leaf sum of squares of [x0, x1] is fma(x1, x1, x0*x0): check both
    roundings against exact rationals (fused) and the two-rounding variant."""
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4000, 2)).astype(np.float32) * np.float32(3.0)
    _, q_fused = oracle.reduce(x, "row", leaf_len=2, sq_fused=True)
    _, q_unf = oracle.reduce(x, "row", leaf_len=2, sq_fused=False)
    differ = 0
    for i in range(x.shape[0]):
        a, b = f32_value(x[i, 0]), f32_value(x[i, 1])
        p0 = round_f32(a * a)
        fused = round_f32(f32_value(p0) + b * b)
        unf = round_f32(f32_value(p0) + f32_value(round_f32(b * b)))
        assert q_fused[i] == fused and q_unf[i] == unf
        differ += fused != unf
    assert differ > 0  # the two readings are distinguishable on this data
