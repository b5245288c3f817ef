"""Pins for the oracle's GEMM walk, split-K cuts and partial combine."""
import os

import numpy as np
import pytest

import oracle
import synth
from exact import all_tree_values, all_trees, catalan, eval_tree, pairwise_recursive, tree_index
from gpu_util import profile

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ONE = 0x3F80  # bf16 1.0

MODELS = {
    "E16": oracle.family_e(16),
    "B16n1": oracle.family_b(16, 1),
    "B8n1": oracle.family_b(8, 1),
    "B16n2": oracle.family_b(16, 2),
    "E4chain": dict(oracle.family_e(16), group=4),
}


def desc(model, S=1, out="fp32", cuts=None, mfma="F32_32X32X16_BF16", combine="BALANCED_NEIGHBOURS_FIRST"):
    d = {"mfma": mfma, "mfma_model": model, "split_k": S, "out_type": out, "combine": combine}
    if cuts is not None:
        d["cut_rule"] = "EXPLICIT"
        d["cuts"] = cuts
    return d


def _read_golden(name):
    meta, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            if parts[0][0].isalpha():
                meta[parts[0]] = parts[1:]
            else:
                rows.append(parts)
    return meta, rows


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(MODELS))
@pytest.mark.parametrize("K", [16, 24, 40])
def test_small_integer_gemm_is_exact(name, K):
    """The K=16 small-integer workload (entries in {-4..4}) and ragged K with a
    zero-padded short last turn: every model returns the exact integer."""
    A, B = synth.gemm_small_int(K=K)
    C = oracle.gemm_bf16(desc(MODELS[name]), A, B)
    exact = synth.bf16_bits_to_f32(A).astype(np.int64) @ synth.bf16_bits_to_f32(B).astype(np.int64).T
    assert np.array_equal(C.astype(np.int64), exact)
    # a transposed operand would give a different answer on this data
    assert not np.array_equal(exact[:, :32], exact[:, :32].T)


@pytest.mark.parametrize("name", ["E16", "B16n1", "B8n1"])
@pytest.mark.parametrize("K,S", [(512, 1), (512, 2), (9728, 1), (9728, 2), (9728, 4),
                                 (9728, 8), (9728, 16), (600, 2), (1000, 3)])
def test_all_ones_counts_every_k(name, K, S):
    """All-ones A and B: every output is exactly K for any split, since each
    1x1 product is exact and every partial and merge stays below 2^24
    ('Taming', appendix D: the count of summed k)."""
    A = np.full((3, K), ONE, dtype=np.uint16)
    B = np.full((5, K), ONE, dtype=np.uint16)
    C = oracle.gemm_bf16(desc(MODELS[name], S=S), A, B)
    assert np.all(C == K)


# ---------------------------------------------------------------------------
# the printed K = 576 span walk
# ---------------------------------------------------------------------------
def _span_walk(model, meta):
    K = int(meta["K"][0])
    cuts = [int(c) for c in meta["cuts"][0].split(",")]
    L = np.float32(float(meta["L"][0]))
    r = np.float32(2.0 ** int(meta["r_log2"][0]))
    ms = np.arange(1, K - 1)
    A = np.zeros((len(ms), K), dtype=np.uint16)
    A[:, 0] = synth.f32_to_bf16_bits(r)
    A[np.arange(len(ms)), ms] = synth.f32_to_bf16_bits(L)
    A[np.arange(len(ms)), ms + 1] = synth.f32_to_bf16_bits(-L)
    B = np.full((1, K), ONE, dtype=np.uint16)
    C = oracle.gemm_bf16(desc(model, S=len(cuts) - 1, cuts=cuts), A, B)[:, 0]
    return ms, C, r


@pytest.mark.parametrize("name", ["B16n1", "B8n1"])
def test_printed_span_walk_k576(name):
    """'Taming', section 4: a truncating instruction whose window cannot hold r
    (r lies 25 binades under L) reproduces the printed walk exactly: 0 for
    m = 1..191, r from 192 on, 0 again at m = 383 alone."""
    meta, rows = _read_golden("splitk_span_walk_k576.txt")
    ms, C, r = _span_walk(MODELS[name], meta)
    expect = np.empty_like(C)
    for lo, hi, v in rows:
        sel = (ms >= int(lo)) & (ms <= int(hi))
        expect[sel] = r if v == "r" else 0.0
    assert np.array_equal(C, expect)


def test_span_walk_tells_models_apart():
    """Under the exact-sum instruction a pair inside one instruction cancels
    before the rounding and r survives, so the printed walk is NOT what
    family E with contiguous slots gives: the walk has power to separate
    them."""
    meta, _ = _read_golden("splitk_span_walk_k576.txt")
    ms, C, r = _span_walk(MODELS["E16"], meta)
    assert C[ms == 1][0] == r          # pair (1,2) shares r's instruction
    assert C[ms == 15][0] == 0.0       # pair (15,16) straddles an instruction
    assert C[ms == 383][0] == 0.0      # pair straddles the split cut


# ---------------------------------------------------------------------------
# one instruction, cut rule, combine
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(MODELS))
def test_single_instruction_gemm_is_the_model(name):
    """K = instruction_k, S = 1: the walk is one instruction from +0."""
    A = synth.bf16_spread(11, (4, 16), -20, 20)
    B = synth.bf16_spread(12, (6, 16), -20, 20)
    C = oracle.gemm_bf16(desc(MODELS[name]), A, B)
    for m in range(4):
        for n in range(6):
            assert C[m, n] == np.float32(oracle.mfma_bf16(MODELS[name], 0.0, A[m], B[n]))


@pytest.mark.parametrize("which", ["measured", "E16"])
def test_one_instruction_is_no_plain_tree(which):
    """K = 8 inside one instruction (the other eight products zero, which
    are neutral): the instruction's result against every ordered fp32
    addition tree over the accumulator and the eight exact products (1430
    trees).  On exponent-spread draws no single tree gives the instruction's
    bits on every draw -- the measured two-stage instruction and the pages'
    exact-sum instruction are not plain fp32 summations -- while on small
    integers every tree and the instruction agree (all exact)."""
    model = MODELS["E16"] if which == "E16" else profile()["models"]["F32_32X32X16_BF16"]
    same_all = np.ones(catalan(8), dtype=bool)
    for draw in range(60):
        a = synth.bf16_spread(3000 + draw, (16,), -12, 12)
        b = synth.bf16_spread(4000 + draw, (16,), -12, 12)
        a[8:] = 0
        acc = synth.f32_spread(5000 + draw, (1,), -12, 12)[0]
        got = np.float32(oracle.mfma_bf16(model, acc, a, b))
        prods = (synth.bf16_bits_to_f32(a[:8]).astype(np.float64) *
                 synth.bf16_bits_to_f32(b[:8]).astype(np.float64)).astype(np.float32)  # exact in fp32
        same_all &= all_tree_values(np.concatenate([[acc], prods]).astype(np.float32)) == got
    assert not same_all.any()
    ai = synth.f32_to_bf16_bits(np.arange(-4, 4, dtype=np.float32).repeat(2))
    bi = synth.f32_to_bf16_bits(np.arange(16, dtype=np.float32) % 5 - 2)
    ai[8:] = 0
    got = np.float32(oracle.mfma_bf16(model, np.float32(3.0), ai, bi))
    prods = synth.bf16_bits_to_f32(ai[:8]) * synth.bf16_bits_to_f32(bi[:8])
    assert (all_tree_values(np.concatenate([[np.float32(3.0)], prods]).astype(np.float32)) == got).all()


def test_walk_chains_instructions_in_ascending_k():
    """K = 48: three instructions from +0, each feeding the next."""
    model = MODELS["B16n1"]
    A = synth.bf16_spread(21, (3, 48), -20, 20)
    B = synth.bf16_spread(22, (3, 48), -20, 20)
    C = oracle.gemm_bf16(desc(model), A, B)
    for m in range(3):
        for n in range(3):
            acc = 0.0
            for k0 in (0, 16, 32):
                acc = oracle.mfma_bf16(model, acc, A[m, k0:k0 + 16], B[n, k0:k0 + 16])
            assert C[m, n] == np.float32(acc)


def test_cut_rule_unit256_remainder_last():
    """span = floor(K/(256 S)) * 256, the remainder in the last split."""
    K = 9728
    spans = {S: np.diff(oracle.split_cuts(K, S)).tolist() for S in (1, 2, 4, 8, 16)}
    assert spans[1] == [9728]
    assert spans[2] == [4864, 4864]
    assert spans[4] == [2304, 2304, 2304, 2816]
    assert spans[8] == [1024] * 7 + [2560]
    assert spans[16] == [512] * 15 + [2048]
    assert oracle.split_cuts(512, 2) == [0, 256, 512]
    assert oracle.split_cuts(700, 2) == [0, 256, 700]
    assert oracle.split_cuts(16, 1) == [0, 16]
    with pytest.raises(ValueError):
        oracle.split_cuts(256, 2)  # a span would be empty


def _level_pairs_tree(lo, hi):
    """Neighbours-first pairing built level by level as an expression tree,
    odd element carried up; an independent construction of the combine's
    shape."""
    level = list(range(lo, hi))
    while len(level) > 1:
        nxt = [(level[i], level[i + 1]) for i in range(0, len(level) - 1, 2)]
        if len(level) % 2:
            nxt.append(level[-1])
        level = nxt
    return level[0]


@pytest.mark.parametrize("S", [2, 3, 4, 5, 6, 7, 8])
def test_combine_is_the_balanced_member_of_all_trees(S):
    """Every ordered binary tree over S exponent-spread partials is evaluated;
    the oracle's combine equals the balanced neighbours-first member, equals
    textbook recursive pairwise summation when S is a power of two, and every
    other tree gives other bits on at least one draw (so a wrong shape would
    be caught by these draws)."""
    trees = all_trees(0, S)
    mine = _level_pairs_tree(0, S)
    caught = np.zeros(len(trees), dtype=bool)
    for draw in range(40):
        vals = synth.f32_spread(1000 + 97 * S + draw, (S,), -12, 12)
        got = np.float32(oracle.tree_balanced(vals))
        assert got == eval_tree(mine, vals)
        if S & (S - 1) == 0:
            assert got == pairwise_recursive(vals)
        results = np.array([eval_tree(t, vals) for t in trees], dtype=np.float32)
        assert np.any(results == got)
        caught |= results != got
    others = [i for i, t in enumerate(trees) if t != mine]
    assert caught[others].all()


@pytest.mark.parametrize("S", [11, 12, 16])
def test_combine_is_the_balanced_member_of_all_trees_up_to_16(S):
    """The same check for split counts up to 16, where the trees are too many
    to build one by one (9,694,845 at S = 16): every tree's fp32 value is
    computed by intervals, the oracle's combine equals the balanced
    neighbours-first member's value, and over 80 exponent-spread draws every
    other tree gives other bits at least once."""
    mine = tree_index(_level_pairs_tree(0, S), 0, S)
    caught = np.zeros(catalan(S - 1), dtype=bool)
    for draw in range(80):
        vals = synth.f32_spread(1000 + 97 * S + draw, (S,), -12, 12)
        allv = all_tree_values(vals)
        got = np.float32(oracle.tree_balanced(vals))
        assert allv[mine] == got, draw
        caught |= allv != got
    assert not caught[mine] and int(caught.sum()) == len(caught) - 1


@pytest.mark.parametrize("S", [2, 4, 8])
def test_gemm_partials_and_combine(S):
    """Each split starts from +0 over its own cut range, and the output is the
    balanced combine of the fp32 partials, rounded once to the output type."""
    model = MODELS["B16n1"]
    K = 256 * S + 48
    a = synth.bf16_spread(51, (K,), -10, 10)
    b = synth.bf16_spread(52, (K,), -10, 10)
    v, parts = oracle.gemm_partials(desc(model, S=S), a, b)
    cuts = oracle.split_cuts(K, S)
    for s in range(S):
        one = oracle.gemm_partials(desc(model, S=1), a[cuts[s]:cuts[s + 1]], b[cuts[s]:cuts[s + 1]])[0]
        assert parts[s] == np.float32(one)
    assert v == np.float32(oracle.tree_balanced(parts))
    vb = oracle.gemm_bf16(desc(model, S=S, out="bf16"), a[None], b[None])[0, 0]
    assert vb == oracle.bf16_rne(np.float32(v))


def test_balanced_and_sequential_merges_differ_at_s4():
    """Sensitivity of the combine: on spread inputs the sequential merge
    (p0+p1)+p2)+p3 and the balanced (p0+p1)+(p2+p3) differ somewhere."""
    model = MODELS["E16"]
    A = synth.bf16_spread(61, (16, 1024), -20, 20)
    B = synth.bf16_spread(62, (16, 1024), -20, 20)
    bal = oracle.gemm_bf16(desc(model, S=4), A, B)
    seq = oracle.gemm_bf16(desc(model, S=4, combine="SEQUENTIAL"), A, B)
    assert np.any(bal != seq)


def test_rows_do_not_depend_on_batch_size():
    """Batch invariance: row i of C is the same for every M > i."""
    model = MODELS["B16n1"]
    X, W = synth.bf16_normal(1003, (64, 256)), synth.bf16_normal(2003, (40, 256), 0.0, 0.02)
    full = oracle.gemm_bf16(desc(model, out="bf16"), X, W)
    for M in (1, 8, 33):
        assert np.array_equal(oracle.gemm_bf16(desc(model, out="bf16"), X[:M], W), full[:M])


def test_points_match_full_output():
    model = MODELS["E16"]
    A, B = synth.gemm_small()
    full = oracle.gemm_bf16(desc(model, S=2, cuts=[0, 256, 512]), A, B)
    rng = np.random.default_rng(1)
    mi = rng.integers(0, 32, 50)
    ni = rng.integers(0, 64, 50)
    pts = oracle.gemm_bf16_points(desc(model, S=2, cuts=[0, 256, 512]), A, B, mi, ni)
    assert np.array_equal(pts, full[mi, ni])


# ---------------------------------------------------------------------------
# the oracle reads the descriptor JSON the library reads
# ---------------------------------------------------------------------------
def _profile():
    import json as _json
    import os as _os
    path = _os.path.join(_os.path.dirname(_os.path.dirname(_os.path.abspath(__file__))),
                         "fixed_order_fp_amd", "profiles", "gfx950.json")
    with open(path) as f:
        return _json.load(f)


def test_oracle_reads_descriptor_json():
    """The same record text gives the oracle the spec it is otherwise handed
    as a dict: equal results on a small split GEMM; refusals of what it does
    not emulate and of another profile's hash."""
    prof = _profile()
    text = ('{"gemm": {"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 256, 512], "out_type": "fp32", '
            '"mfma_profile_hash": "0x%016x"}}' % oracle.profile_models_hash(prof))
    g, r = oracle.desc_from_json(text, prof)
    assert r is None and g["split_k"] == 2 and g["cuts"] == [0, 256, 512]
    A, B = synth.gemm_small()
    direct = {"mfma": "F32_32X32X16_BF16", "mfma_model": prof["models"]["F32_32X32X16_BF16"], "split_k": 2,
              "cut_rule": "EXPLICIT", "cuts": [0, 256, 512], "out_type": "fp32"}
    assert np.array_equal(oracle.gemm_bf16(g, A, B).view(np.uint32), oracle.gemm_bf16(direct, A, B).view(np.uint32))
    _, rd = oracle.desc_from_json('{"reduce": {"axis": "col", "sq_fma": "unfused"}}', prof)
    assert rd["axis"] == "col" and rd["sq_fused"] is False
    for bad in ('{"gemm": {"acc_update": "SEPARATE_ADD"}}', '{"gemm": {"k_slot_layout": "STRIDED"}}',
                '{"gemm": {"mfma_profile_hash": "0x0000000000000001"}}', '{"gemm": {"tile": 1}}',
                '{"reduce": {"tree": "SEQUENTIAL"}}', '{"other": {}}'):
        with pytest.raises(ValueError):
            oracle.desc_from_json(bad, prof)
