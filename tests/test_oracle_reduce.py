"""Pins for the oracle's fixed-order reductions: leaves folded in index order
with no seed, a balanced neighbours-first tree over the leaves
('Taming Bitwise Behavior', sections 3.1 and 5.1)."""
import math
import os

import numpy as np
import pytest

import oracle
import synth
from exact import all_tree_values, all_trees, catalan, eval_tree, pairwise_recursive, tree_index

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            p = line.split()
            (meta.__setitem__(p[0], p[1:]) if p[0][0].isalpha() else rows.append(p))
    return meta, rows


def test_printed_contiguous_grouping_walk():
    """'Taming' section 4 (i): eight terms in two sequential groups of four;
    r at 0, the cancelling pair walked; printed outcomes 0, 0, 0, r."""
    meta, rows = _golden("contiguous_grouping_walk.txt")
    n, g = int(meta["n"][0]), int(meta["group"][0])
    L, r = np.float32(float(meta["L"][0])), np.float32(2.0 ** int(meta["r_log2"][0]))
    for p, expect in rows:
        p = int(p)
        x = np.zeros((1, n), dtype=np.float32)
        x[0, int(meta["r_index"][0])] = r
        x[0, p], x[0, p + 1] = L, -L
        s, _ = oracle.reduce(x, "row", leaf_len=g)
        assert s[0] == (r if expect == "r" else 0.0), p


def test_printed_strided_grouping_walk():
    """'Taming' section 4 (ii): the strided grouping {0,2,4,6} + {1,3,5,7} is the
    contiguous grouping of the permuted terms; printed outcomes: r absorbed at
    2 and 4, surviving at 1, 3, 5, 7."""
    meta, rows = _golden("strided_grouping_walk.txt")
    groups = [list(map(int, g.split(","))) for g in meta["groups"]]
    perm = [i for grp in groups for i in grp]
    L, r = np.float32(float(meta["L"][0])), np.float32(2.0 ** int(meta["r_log2"][0]))
    for idx, expect in rows:
        x = np.zeros(8, dtype=np.float32)
        x[int(meta["plus_L_index"][0])] = L
        x[int(meta["minus_L_index"][0])] = -L
        x[int(idx)] = r
        s, _ = oracle.reduce(x[perm][None], "row", leaf_len=len(groups[0]))
        assert s[0] == (r if expect == "r" else 0.0), idx


def _expected_tree(n, leaf_len):
    """Independent construction of the reduction's dependence tree: each leaf
    a left fold over its consecutive indices, the leaves paired neighbours
    first, level by level, an odd one carried up."""
    leaves = []
    for j0 in range(0, n, leaf_len):
        t = j0
        for j in range(j0 + 1, min(j0 + leaf_len, n)):
            t = (t, j)
        leaves.append(t)
    level = leaves
    while len(level) > 1:
        nxt = [(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


@pytest.mark.parametrize("n,leaf", [(4, 1), (6, 2), (7, 2), (8, 2), (8, 4), (9, 4), (10, 3)])
def test_reduction_is_one_member_of_all_trees(n, leaf):
    """Brute force at small n: the oracle's sum equals the stated tree, and
    every other ordered tree differs on some exponent-spread draw."""
    trees = all_trees(0, n)
    mine = _expected_tree(n, leaf)
    caught = np.zeros(len(trees), dtype=bool)
    for draw in range(60):
        x = synth.f32_spread(500 + 13 * n + leaf + draw, (1, n), -12, 12)
        s, _ = oracle.reduce(x, "row", leaf_len=leaf)
        assert s[0] == eval_tree(mine, x[0])
        caught |= np.array([eval_tree(t, x[0]) for t in trees], dtype=np.float32) != s[0]
    assert caught[[i for i, t in enumerate(trees) if t != mine]].all()


@pytest.mark.parametrize("n,leaf", [(16, 1), (16, 2), (16, 4), (16, 8), (16, 16), (13, 4), (14, 3)])
def test_reduction_is_one_member_of_all_trees_up_to_16(n, leaf):
    """The same at n up to 16 (9,694,845 ordered trees at n = 16), every
    tree's fp32 value computed by intervals: the oracle's sum equals its
    stated tree's value, and over 80 exponent-spread draws every other tree
    gives other bits at least once."""
    mine = tree_index(_expected_tree(n, leaf), 0, n)
    caught = np.zeros(catalan(n - 1), dtype=bool)
    for draw in range(80):
        x = synth.f32_spread(700 + 13 * n + leaf + draw, (1, n), -12, 12)
        s, _ = oracle.reduce(x, "row", leaf_len=leaf)
        allv = all_tree_values(x[0])
        assert allv[mine] == s[0], draw
        caught |= allv != s[0]
    assert not caught[mine] and int(caught.sum()) == len(caught) - 1


def test_one_leaf_is_a_sequential_fold():
    """leaf_len = n: a left fold, which numpy's add.accumulate computes."""
    x = synth.f32_spread(9, (5, 100), -15, 15)
    s, _ = oracle.reduce(x, "row", leaf_len=100)
    for i in range(5):
        assert s[i] == np.add.accumulate(x[i])[-1]


@pytest.mark.parametrize("p", [1, 3, 6, 8])
def test_unit_leaves_are_textbook_pairwise(p):
    """leaf_len = 1, n = 2^p: recursive pairwise summation."""
    x = synth.f32_spread(10 + p, (4, 2 ** p), -15, 15)
    s, _ = oracle.reduce(x, "row", leaf_len=1)
    for i in range(4):
        assert s[i] == pairwise_recursive(x[i])


def test_all_ones_and_small_integers_are_exact():
    x = np.ones((3, 8192), dtype=np.float32)
    s, q = oracle.reduce(x, "row")
    assert np.all(s == 8192) and np.all(q == 8192)
    rng = np.random.default_rng(4)
    xi = rng.integers(-50, 51, size=(6, 1000)).astype(np.float32)
    s, q = oracle.reduce(xi, "row")
    assert np.array_equal(s.astype(np.int64), xi.astype(np.int64).sum(1))
    assert np.array_equal(q.astype(np.int64), (xi.astype(np.int64) ** 2).sum(1))
    ci = synth.f32_to_bf16_bits(xi.T.copy())  # column sum of bf16 integers
    s, q = oracle.reduce(ci, "col", in_type="bf16")
    assert np.array_equal(s.astype(np.int64), xi.astype(np.int64).sum(1))


def test_column_axis_is_row_axis_of_the_transpose():
    y = synth.bf16_normal(2002, (300, 40), 0.0, 0.1)
    sc, qc = oracle.reduce(y, "col", in_type="bf16")
    sr, qr = oracle.reduce(synth.bf16_bits_to_f32(y).T.copy(), "row")
    assert np.array_equal(sc, sr) and np.array_equal(qc, qr)


def test_short_last_leaf_and_odd_leaf_count():
    """n = 100 with leaves of 32: leaves of 32, 32, 32, 4; n = 70: 32, 32, 6
    (three leaves, the third carried up)."""
    for n in (100, 70):
        x = synth.f32_spread(n, (2, n), -10, 10)
        s, _ = oracle.reduce(x, "row")
        for i in range(2):
            assert s[i] == eval_tree(_expected_tree(n, 32), x[i])


def test_fused_and_unfused_squares_are_both_modelled():
    x = synth.f32_normal(1002, (64, 8192))
    _, qf = oracle.reduce(x, "row", sq_fused=True)
    _, qu = oracle.reduce(x, "row", sq_fused=False)
    assert np.any(qf != qu)


def test_free_order_error_bound_holds_for_the_oracle():
    """Any summation order obeys |y - sum| <= gamma_{n-1} sum |x|
    (gamma_k = k u / (1 - k u), u = 2^-24); math.fsum gives the exact sum."""
    x = synth.f32_normal(1002, (32, 8192))
    s, _ = oracle.reduce(x, "row")
    u = 2.0 ** -24
    n = x.shape[1]
    g = (n - 1) * u / (1 - (n - 1) * u)
    for i in range(x.shape[0]):
        exact = math.fsum(x[i].astype(np.float64))
        assert abs(float(s[i]) - exact) <= g * float(np.abs(x[i].astype(np.float64)).sum())
