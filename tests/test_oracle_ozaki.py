"""Pins for the oracle's Ozaki-scheme GEMM ("GPU Mechanism", the exact-GEMM
paragraph and intervention (a): each operand row scaled by a frexp power of
two and cut into four signed 7-bit pieces, the piece products exact integers,
their fp64 sum taken in a set order and rounded once).  Each check is a fact the scheme fixes: the
slices rebuild the rows they came from, integer accumulation makes the result
independent of the k order, inputs the slices hold exactly give the exactly
rounded product, power-of-two row scaling passes straight through, and the
single rounding from fp64 to bf16 is not a rounding through fp32."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def exact_rounded_f32(a_row, b_row):
    """sum_k a_k b_k as an exact fraction, rounded once to float32."""
    s = sum(Fraction(float(x)) * Fraction(float(y)) for x, y in zip(a_row, b_row))
    return np.float32(float(s)) if s == 0 else _rne32(s)


def _rne32(fr):
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - 23)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return np.float32(sign * float(q * ulp))


def test_slices_rebuild_rows_they_hold():
    """A row whose elements all lie within 28 bits below its largest is cut
    exactly: sum_s q_s 2^(-7(s+1)) 2^e gives it back, every q_s in [-127, 127]."""
    rng = np.random.default_rng(1)
    x = (rng.integers(-2 ** 20, 2 ** 20, 300) * 2.0 ** -30).astype(np.float32)
    x[0] = np.float32(2.0 ** -10 * 0.99)  # the largest magnitude
    q, e = oracle.ozaki_slice_row(x)
    assert np.abs(q).max() <= 127
    back = sum(q[s].astype(np.float64) * 2.0 ** (-7 * (s + 1)) for s in range(4)) * 2.0 ** e
    assert np.array_equal(back, x.astype(np.float64))


def test_zero_row_and_signs():
    q, e = oracle.ozaki_slice_row(np.zeros(9, np.float32))
    assert e == 0 and not q.any()
    x = synth.f32_normal(2, (1, 64))[0]
    q1, e1 = oracle.ozaki_slice_row(x)
    q2, e2 = oracle.ozaki_slice_row(-x)
    assert e1 == e2 and np.array_equal(q2, -q1)   # truncation toward zero is odd


def test_small_integers_are_exact():
    """Integer entries up to 127: one slice holds them, every slice product is
    exact and the fp64 sum is exact, so C is the integer product."""
    rng = np.random.default_rng(3)
    A = rng.integers(-127, 128, (20, 200)).astype(np.float32)
    B = rng.integers(-127, 128, (30, 200)).astype(np.float32)
    C = oracle.ozaki_gemm(A, B)
    assert np.array_equal(C.astype(np.int64), A.astype(np.int64) @ B.astype(np.int64).T)


def test_k_order_does_not_matter():
    """Permuting k in both operands leaves every bit: the slice products are
    integers, whose sum has no order."""
    A = synth.f32_spread(4, (16, 333), -8, 8)
    B = synth.f32_spread(5, (24, 333), -8, 8)
    C = oracle.ozaki_gemm(A, B)
    for seed in range(3):
        p = np.random.default_rng(seed).permutation(333)
        Cp = oracle.ozaki_gemm(A[:, p], B[:, p])
        assert np.array_equal(C.view(np.uint32), Cp.view(np.uint32))


def test_held_inputs_give_the_exactly_rounded_product():
    """bf16 entries whose exponents lie within 20 of their row's largest are
    held exactly by the slices; with K small the fp64 sum is exact too, so C
    is the exact dot product rounded once."""
    rng = np.random.default_rng(6)
    A = synth.bf16_spread(7, (6, 24), -10, 10)
    B = synth.bf16_spread(8, (7, 24), -10, 10)
    C = oracle.ozaki_gemm(A, B, in_type="bf16")
    Af, Bf = synth.bf16_bits_to_f32(A), synth.bf16_bits_to_f32(B)
    for m in range(6):
        for n in range(7):
            assert C[m, n] == exact_rounded_f32(Af[m], Bf[n])
    del rng


def test_power_of_two_row_scaling_passes_through():
    A = synth.f32_normal(9, (8, 128))
    B = synth.f32_normal(10, (9, 128))
    C = oracle.ozaki_gemm(A, B)
    for j in (-7, 3, 20):
        Cs = oracle.ozaki_gemm(np.ldexp(A, j).astype(np.float32), B)
        assert np.array_equal(Cs, np.ldexp(C, j).astype(np.float32))


def test_accuracy_is_fp32_class():
    """Against a float64 product: within a few units of 2^-28 of sum |a||b|
    (what the slices drop) plus the final rounding."""
    A = synth.f32_normal(11, (32, 1000))
    B = synth.f32_normal(12, (40, 1000))
    C = oracle.ozaki_gemm(A, B).astype(np.float64)
    ref = A.astype(np.float64) @ B.astype(np.float64).T
    bound = np.abs(A).astype(np.float64) @ np.abs(B).astype(np.float64).T * 2.0 ** -26 + np.abs(ref) * 2.0 ** -24
    assert np.all(np.abs(C - ref) <= bound)


def test_one_rounding_to_bf16():
    """From fp64 to bf16 in one step: equal to torch's fp32 -> bf16 cast for
    values that are floats, and different from a rounding through fp32 where
    that second rounding would land on a tie."""
    rng = np.random.default_rng(13)
    f = (rng.standard_normal(2000) * np.exp(rng.uniform(-40, 40, 2000))).astype(np.float32)
    f[:4] = [np.float32(1e-40), np.float32(-3e38), np.float32(0.0), np.float32(-0.0)]
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_from_f64(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, want)
    v = 1.0 + 2.0 ** -8 + 2.0 ** -40   # just above the bf16 tie between 1 and 1 + 2^-7
    assert oracle.bf16_from_f64(v) == 0x3F81          # one rounding: up
    assert oracle.bf16_from_f64(float(np.float32(v))) == 0x3F80   # through fp32 it would tie down to even
    assert oracle.bf16_from_f64(3.5e38) == 0x7F80     # past the largest bf16: infinity


# ---------------------------------------------------------------------------
# The fp64 order of the 16 slice products.  Every row below is built from
# chosen base-128 digits (an element is 2^e sum_s q_s 128^-(s+1) with the row
# exponent e = 0), one nonzero digit per element, so that column k adds
# qa_s qb_t to exactly one slice product acc[s][t].  The products are then
# placed so that the exact dot product lies on an fp32 (or bf16) rounding
# midpoint plus a remainder far below the fp64 precision of the partial sums:
# which remainder survives the fp64 additions decides the final rounding,
# so the stated order (s + t from 6 down to 0, s ascending within a level)
# is told apart from the reversed level walk and from s descending.
# ---------------------------------------------------------------------------
def _digits_row(cols):
    """Elements from digit tuples (q0, q1, q2, q3), all digits of one sign."""
    return np.array([sum(q * 2.0 ** (-7 * (s + 1)) for s, q in enumerate(d)) for d in cols],
                    dtype=np.float32)


def _fill(acc_target, s, t, sign=1):
    """Columns (digit tuple of a, digit tuple of b) whose products sum to
    acc_target in acc[s][t]: as many 127 x 127 as fit, then 127 x r, then 1 x r."""
    cols, left = [], acc_target
    one = lambda pos, q: tuple(q if i == pos else 0 for i in range(4))
    while left >= 127 * 127:
        cols.append((one(s, 127), one(t, 127 * sign)))
        left -= 127 * 127
    if left >= 127:
        cols.append((one(s, left // 127), one(t, 127 * sign)))
        left -= (left // 127) * 127
    if left:
        cols.append((one(s, 1), one(t, left * sign)))
    return cols


def _rows(spec):
    cols = [c for (s, t, acc) in spec for c in _fill(abs(acc), s, t, 1 if acc > 0 else -1)]
    # an anchor column holding each row's largest magnitude 127/128 (row
    # exponent 0) whose products land in acc[0][0] only through b = 0
    cols.append(((127, 0, 0, 0), (0, 0, 0, 0)))
    cols.append(((0, 0, 0, 0), (127, 0, 0, 0)))
    a = _digits_row([c[0] for c in cols])
    b = _digits_row([c[1] for c in cols])
    return a, b


def _round_bits(fr, keep):
    """Fraction -> nearest number with `keep` significant bits, ties to even
    (written from the definition of round-to-nearest-even)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - keep + 1)
    q, r = divmod(a, ulp)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def _order_sum(acc, order):
    """Sequential sum of acc[s][t] 2^(-7(s+t+2)) in `order`, each add rounded
    to 53 bits."""
    v = Fraction(0)
    for s, t in order:
        v = _round_bits(v + Fraction(acc[s][t]) * Fraction(2) ** (-7 * (s + t + 2)), 53)
    return v


STATED = [(s, lev - s) for lev in range(6, -1, -1) for s in range(4) if 0 <= lev - s <= 3]
LEVELS_UP = [(s, lev - s) for lev in range(0, 7) for s in range(4) if 0 <= lev - s <= 3]
S_DESC = [(s, lev - s) for lev in range(6, -1, -1) for s in range(3, -1, -1) if 0 <= lev - s <= 3]


def _acc_of(spec):
    acc = [[0] * 4 for _ in range(4)]
    for s, t, v in spec:
        acc[s][t] += v
    return acc


@pytest.mark.parametrize("case", ["levels_fp32", "levels_bf16", "s_order_fp32"])
def test_fp64_recombination_order_is_pinned(case):
    """The stated fp64 order gives bits that the reversed level walk (case
    levels_*) or s descending within a level (case s_order) would not."""
    if case == "levels_fp32":
        # 2^6 + 2^-18 (an fp32 midpoint) + 6 2^-49: the two 3 2^-49 pieces,
        # summed first, survive the add of 2^6 (0.75 of its fp64 ulp);
        # added one by one after it they are each lost (0.375 ulp)
        spec, out, want = [(0, 0, 2 ** 20), (0, 1, 8), (2, 3, 3), (3, 2, 3)], "fp32", 64 + 2.0 ** -17
    elif case == "levels_bf16":
        # 2^6 + 2^-2 (a bf16 midpoint) + 6 2^-49, the same way to 64.5
        spec, out, want = [(0, 0, 2 ** 20 + 2 ** 12), (2, 3, 3), (3, 2, 3)], "bf16", 64.5
    else:
        # T01 = 1/2, T10 = -(1/2 - 2^-21), carried 2^-45 + 3 2^-56: with T01
        # first the 3 2^-56 is lost (0.375 of the ulp of 1/2) and the result
        # 2^-21 + 2^-45 is an fp32 midpoint going to the even 2^-21; with T10
        # first it is rounded up to 2^-54 (0.75 of the ulp below 1/2) and
        # the result rounds up to 2^-21 + 2^-44
        spec, out, want = [(0, 1, 2 ** 20), (1, 0, -(2 ** 20 - 1)), (2, 3, 16), (3, 3, 3)], "fp32", 2.0 ** -21
    a, b = _rows(spec)
    # the premise: the oracle cuts these rows into the designed digits
    qa, ea = oracle.ozaki_slice_row(a)
    qb, eb = oracle.ozaki_slice_row(b)
    assert ea == 0 and eb == 0
    acc = _acc_of(spec)
    got_acc = qa.astype(np.int64) @ qb.astype(np.int64).T
    assert got_acc.tolist() == acc
    keep = 24 if out == "fp32" else 8
    stated = _round_bits(_order_sum(acc, STATED), keep)
    other = _order_sum(acc, LEVELS_UP if case.startswith("levels") else S_DESC)
    assert stated == Fraction(want)
    assert _round_bits(other, keep) != stated       # the order is visible here
    res = oracle.ozaki_gemm(a[None, :], b[None, :], in_type="fp32", out_type=out)
    if out == "fp32":
        assert res[0, 0] == np.float32(want)
    else:
        assert int(res[0, 0]) == int(oracle.bf16_rne(np.array([want], np.float32))[0])
