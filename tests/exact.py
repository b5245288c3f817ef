"""Exact-arithmetic references written independently of the oracle (Python
Fractions and big integers).  They are the things the oracle is pinned to:
correct rounding from the IEEE-754 definition, the exact value of a bf16 /
fp32 bit pattern, and the two instruction models as the pages state them in
words.
"""
from fractions import Fraction
import math
import struct

import numpy as np

F32_MAX = Fraction((2 ** 24 - 1) * 2 ** 104)


def bf16_value(h):
    """Exact value of a bf16 bit pattern (finite only)."""
    h = int(h)
    s = -1 if h >> 15 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    assert e != 0xFF
    if e == 0:
        return s * Fraction(f, 2 ** 133)
    return s * Fraction(128 + f, 128) * Fraction(2) ** (e - 127)


def f32_value(x):
    x = float(np.float32(x))
    assert math.isfinite(x)
    return Fraction(x)


def _floor_log2(q):
    """floor(log2(q)) for a positive Fraction."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_float(q, prec, emin, emax, mode="rne"):
    """Round the exact rational q to a binary format with `prec` significand
    bits and normal exponents [emin, emax], by the IEEE-754 definition: the
    nearest representable value, ties to the even significand (rne), or the
    one nearer zero (rz).  Returns a Fraction, or +-inf as a float."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    ulp = Fraction(2) ** (e - (prec - 1))
    n = a / ulp
    k = n.numerator // n.denominator
    rem = n - k
    if mode == "rne":
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
            k += 1
    elif mode != "rz":
        raise ValueError(mode)
    v = k * ulp
    top = Fraction(2) ** (emax + 1)
    if v >= top:
        if mode == "rz":
            return sign * (top - Fraction(2) ** (emax - prec + 1))
        return sign * math.inf
    return sign * v


def round_f32(q, mode="rne"):
    v = round_float(q, 24, -126, 127, mode)
    return np.float32(float(v))


def round_bf16_bits(q):
    """RNE to bf16, returned as a bit pattern."""
    v = round_float(q, 8, -126, 127, "rne")
    f = np.float32(float(v))
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


# ----------------------------------------------------------------------------
# the two instruction models, restated from the pages
# ----------------------------------------------------------------------------


def family_e_instr(acc, a_bits, b_bits):
    """'Taming', 3.2.1: acc <- acc (+) sum of the instruction's products, the
    sum exact, the one rounding being the fp32 addition itself."""
    s = f32_value(acc) + sum(bf16_value(a) * bf16_value(b) for a, b in zip(a_bits, b_bits))
    return round_f32(s, "rne")


def _bf16_parts(h):
    """(sign, 8-bit integer significand, exponent) with value
    sign * sig * 2^(exp - 7); subnormals use exponent -126 and no hidden bit."""
    h = int(h)
    s = -1 if h >> 15 else 1
    e = (h >> 7) & 0xFF
    f = h & 0x7F
    if e == 0:
        return s, f, -126
    return s, 128 + f, e - 127


def family_b_instr(acc, a_bits, b_bits, nfma, neab):
    """Emulator README, 'Tensor Core Matmul', its four steps, per block of NFMA
    products (blocks chained, each feeding the next as its accumulator):
      1. multiply significands as integers and add exponents, unrounded;
      2. take the max exponent over the block's products and the accumulator;
      3. put every significand on neab extra low bits and align it to that max
         inside a window of 2+23+neab bits, dropping the bits below;
      4. add as integers and truncate to fp32."""
    acc = np.float32(acc)
    for g0 in range(0, len(a_bits), nfma):
        terms = []  # (sign, integer significand with F fraction bits, exponent)
        F = 23 + neab
        for a, b in zip(a_bits[g0:g0 + nfma], b_bits[g0:g0 + nfma]):
            sa, ma, ea = _bf16_parts(a)
            sb, mb, eb = _bf16_parts(b)
            if ma * mb == 0:
                continue
            # product significand has 14 fraction bits; move it to F of them
            terms.append((sa * sb, (ma * mb) << (F - 14), ea + eb))
        if acc != 0:
            u = f32_bits(acc)
            e = (u >> 23) & 0xFF
            m = (u & 0x7FFFFF) | (0x800000 if e else 0)
            terms.append((-1 if u >> 31 else 1, m << (F - 23), (e - 127) if e else -126))
        if not terms:
            acc = np.float32(0.0)
            continue
        emax = max(t[2] for t in terms)
        total = 0
        for s, m, e in terms:
            total += s * (m >> (emax - e))  # bits below the window are dropped
        acc = round_f32(Fraction(total) * Fraction(2) ** (emax - F), "rz")
    return acc


# ----------------------------------------------------------------------------
# trees
# ----------------------------------------------------------------------------


def all_trees(lo, hi):
    """Every ordered binary tree over leaves lo..hi-1 (Catalan many)."""
    if hi - lo == 1:
        return [lo]
    out = []
    for mid in range(lo + 1, hi):
        for L in all_trees(lo, mid):
            for R in all_trees(mid, hi):
                out.append((L, R))
    return out


def eval_tree(t, vals):
    """Evaluate a tree with float32 additions (numpy scalars round to fp32)."""
    if isinstance(t, int):
        return np.float32(vals[t])
    return np.float32(eval_tree(t[0], vals) + eval_tree(t[1], vals))


def pairwise_recursive(vals):
    """Textbook recursive pairwise summation for a power-of-two count: the sum
    of the first half plus the sum of the second half."""
    n = len(vals)
    if n == 1:
        return np.float32(vals[0])
    assert n % 2 == 0
    return np.float32(pairwise_recursive(vals[: n // 2]) + pairwise_recursive(vals[n // 2:]))


def two_stage_instr(acc, a_bits, b_bits, group, F, G):
    """The two-stage placement of the accumulator, restated with rationals:
    per group of products (chained in slot order):
      1. e_ref = the largest raw product exponent (ea + eb) of the group;
         every product keeps only its bits at or above 2^(e_ref - F), the
         magnitude truncated (toward zero);
      2. the accumulator is cut at the same bit, its two's complement
         truncated (toward -inf);
      3. everything is summed exactly; the sum keeps only its bits at or
         above 2^(e_lead - G), e_lead its leading bit, two's complement
         truncated (toward -inf);
      4. one round-to-nearest-even to fp32.
    A group without a nonzero product leaves the accumulator as it is, except
    that a -0 accumulator comes out +0 (the sum of step 3 is an integer
    multiple of 2^lsb, which has no negative zero)."""
    acc = np.float32(acc)

    def cut(v, lsb, floor):
        q = v / lsb
        if floor or v >= 0:
            k = q.numerator // q.denominator
        else:
            k = -((-q.numerator) // q.denominator)
        return k * lsb

    for g0 in range(0, len(a_bits), group):
        prods = []
        for a, b in zip(a_bits[g0:g0 + group], b_bits[g0:g0 + group]):
            _, ma, ea = _bf16_parts(a)
            _, mb, eb = _bf16_parts(b)
            v = bf16_value(a) * bf16_value(b)
            if v != 0:
                prods.append((v, ea + eb))
        if not prods:
            if acc == 0:
                acc = np.float32(0.0)
            continue
        eref = max(e for _, e in prods)
        lsb = Fraction(2) ** (eref - F)
        s = sum(cut(v, lsb, False) for v, _ in prods) + cut(f32_value(acc), lsb, True)
        if s != 0:
            lead = _floor_log2(abs(s))
            s = cut(s, Fraction(2) ** (lead - G), True)
        acc = round_f32(s, "rne") if s != 0 else np.float32(0.0)
    return acc


def catalan(n):
    from math import comb
    return comb(2 * n, n) // (n + 1)


def all_tree_values(vals):
    """fp32 values of every ordered binary tree over vals (Catalan(S-1) of
    them), by intervals: the trees over [i, j) are those over [i, k) joined
    to those over [k, j), k ascending, each pair added in fp32; the array
    order is that enumeration."""
    S = len(vals)
    V = {(i, i + 1): np.array([vals[i]], dtype=np.float32) for i in range(S)}
    for length in range(2, S + 1):
        for i in range(S - length + 1):
            j = i + length
            V[(i, j)] = np.concatenate([(V[(i, k)][:, None] + V[(k, j)][None, :]).ravel() for k in range(i + 1, j)])
    return V[(0, S)]


def tree_index(tree, i, j):
    """Position of one tree over [i, j) in all_tree_values' order."""
    if isinstance(tree, int):
        return 0

    def span(t):
        return (t, t + 1) if isinstance(t, int) else (span(t[0])[0], span(t[1])[1])

    k = span(tree[0])[1]
    off = sum(catalan(kk - i - 1) * catalan(j - kk - 1) for kk in range(i + 1, k))
    return off + tree_index(tree[0], i, k) * catalan(j - k - 1) + tree_index(tree[1], k, j)
