"""Static check of every compiled GEMM variant's accumulation chains (the
AMDGCN the library compiles to, read by tests/isa_tree.py): one matrix instruction, the
descriptor's, accumulating in place; nothing else writing an accumulator in
the k walk; the same number of instructions per accumulator per turn.  The
planted-mistake cases show each check fires on the kind of change that would
move bits (a split accumulator, an extra add, a skipped k block, another
instruction)."""
import re

import pytest

import isa_tree as T

pytestmark = pytest.mark.slow


@pytest.fixture(scope="module")
def gemm_asm():
    return T.device_asm("bg_gemm_bf16.hip")


@pytest.fixture(scope="module")
def w8a8_asm():
    return T.device_asm("bg_w8a8.hip")


def test_every_bf16_gemm_variant(gemm_asm):
    vs = T.gemm_variants(gemm_asm)
    assert len(vs) >= 100  # every tile x output x reduction instantiation
    bad = {name: p for name, lines, i, ks, bl in vs for p in [T.check_kernel(lines, i, ks, bl)] if p}
    assert not bad, bad


def test_every_w8a8_variant(w8a8_asm):
    vs = T.w8a8_variants(w8a8_asm)
    assert len(vs) >= 10
    bad = {name: p for name, lines, i, ks, bl in vs for p in [T.check_kernel(lines, i, ks, bl)] if p}
    assert not bad, bad


def _headline(asm):
    for name, lines, i, ks, bl in T.gemm_variants(asm):
        if "pipe_kernelILi320ELi256ELi2ELi4ELi2ELi1ELi0ELi64E" in name:
            return list(lines), i, ks, bl
    raise AssertionError("headline variant not compiled")


def _mfma_in_loop(lines):
    loop = set(i for idx in T.loops(lines).values() for i in idx)
    return [i for i, l in enumerate(lines) if "v_mfma" in l and i in loop]


def test_planted_split_accumulator_is_caught(gemm_asm):
    lines, i, ks, bl = _headline(gemm_asm)
    j = _mfma_in_loop(lines)[0]
    lines[j] = re.sub(r"(v_mfma\S+\s+)v\[(\d+):(\d+)\]", lambda m: f"{m.group(1)}v[{int(m.group(2)) + 300}:"
                      f"{int(m.group(3)) + 300}]", lines[j], count=1)
    assert any("in place" in p for p in T.check_kernel(lines, i, ks, bl))


def test_planted_add_into_an_accumulator_is_caught(gemm_asm):
    lines, i, ks, bl = _headline(gemm_asm)
    j = _mfma_in_loop(lines)[0]
    acc = lines[j].split()[1].rstrip(",")
    first = re.match(r"v\[(\d+):", acc).group(1)
    lines.insert(j + 1, f"\tv_add_f32_e32 v{first}, v{first}, v0")
    assert any("writes accumulator" in p for p in T.check_kernel(lines, i, ks, bl))


def test_planted_skipped_k_block_is_caught(gemm_asm):
    lines, i, ks, bl = _headline(gemm_asm)
    j = _mfma_in_loop(lines)[0]
    del lines[j]
    assert any("different numbers" in p for p in T.check_kernel(lines, i, ks, bl))


def test_planted_other_instruction_is_caught(gemm_asm):
    lines, i, ks, bl = _headline(gemm_asm)
    j = _mfma_in_loop(lines)[0]
    lines[j] = lines[j].replace("v_mfma_f32_32x32x16_bf16", "v_mfma_f32_32x32x8_bf16")
    assert any("expected" in p for p in T.check_kernel(lines, i, ks, bl))


# ---------------------------------------------------------------------------
# canonical dependence-tree signatures ("Taming Bitwise Behavior", section 6
# and Table 3: the reduction tree read back from the compiled AMDGCN and
# compared across variants and builds)
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def reduce_asm():
    return T.device_asm("bg_reduce.hip")


def _combines(asm):
    return {n: l for n, l in T.kernels(asm).items() if "splitk_combine_kernel" in n and T.template_ints(n)[0] > 0}


def test_split_k_combine_trees_are_the_balanced_tree(gemm_asm):
    """Every compiled split count, fp32 and bf16 output: the loads resolve to
    the planes 0..S-1 once each, and the adds over them form the balanced
    neighbours-first tree the definition gives (the runtime-S loop kernel is
    checked against the oracle at run time only)."""
    cs = _combines(gemm_asm)
    assert len(cs) >= 16
    for name, lines in cs.items():
        S = T.template_ints(name)[0]
        sig = T.combine_tree_signature(lines)
        assert sig is not None, name
        assert sig[1] == list(range(S)), (name, sig)
        assert sig[0] == T.balanced_tree([f"P{i}" for i in range(S)]), (name, sig[0])


def test_row_reduction_trees_are_the_definition(reduce_asm):
    """bf16 and fp32 input, fused and unfused sum of squares: the leaf of 32
    elements folded in index order with no seed, then the count-up wave tree
    (DPP row shifts 1, 2, 4, 8, then (r0 + r1) + (r2 + r3) over the row
    roots), read back from the code."""
    n = 0
    for name, lines in T.kernels(reduce_asm).items():
        if "reduce_row_kernel" not in name:
            continue
        bf16, fused = "ItLb" in name, "Lb1E" in name
        sm, sq = T.leaf_chain(32, fused)
        assert T.row_tree_signature(lines, bf16) == sorted([T.wave_tree(sm), T.wave_tree(sq)]), name
        n += 1
    assert n == 4


def test_gemm_chain_signature_is_one_per_instruction(gemm_asm):
    """Every compiled GEMM variant of one instruction (tile, waves, stages,
    load path, output, split or reduction epilogue) has the same chain
    signature; the two instructions have different ones."""
    per = {}
    for name, lines, i, ks, bl in T.gemm_variants(gemm_asm):
        k_turn = ks * T.INSTR_K[i]
        per.setdefault(i, set()).add(T.gemm_chain_signature(lines, i, k_turn))
    assert per[0] == {"chain[v_mfma_f32_32x32x16_bf16, in place, k step 16, ascending]"}
    assert per[1] == {"chain[v_mfma_f32_16x16x32_bf16, in place, k step 32, ascending]"}


def _signatures(gemm, red):
    out = {}
    for name, lines in _combines(gemm).items():
        out[name] = T.combine_tree_signature(lines)
    for name, lines, i, ks, bl in T.gemm_variants(gemm):
        out[name] = T.gemm_chain_signature(lines, i, ks * T.INSTR_K[i])
    for name, lines in T.kernels(red).items():
        if "reduce_row_kernel" in name:
            out[name] = T.row_tree_signature(lines, "ItLb" in name)
    return out


def test_signatures_equal_across_two_builds(gemm_asm, reduce_asm):
    """A second build at -O2 schedules the code differently; every kernel's
    signature is unchanged."""
    a = _signatures(gemm_asm, reduce_asm)
    b = _signatures(T.device_asm("bg_gemm_bf16.hip", "-O2"), T.device_asm("bg_reduce.hip", "-O2"))
    common = set(a) & set(b)
    assert len(common) >= 150
    diff = {k: (a[k], b[k]) for k in common if a[k] != b[k]}
    assert not diff, diff


def test_planted_combine_reorder_is_caught(gemm_asm):
    """(P0 + P2) + (P1 + P3) in place of (P0 + P1) + (P2 + P3): the first two
    adds of the S = 4 kernel take swapped operands."""
    name, lines = next((n, list(l)) for n, l in _combines(gemm_asm).items() if T.template_ints(n) == [4, 0])
    adds = [k for k, l in enumerate(lines) if "v_add_f32" in l]
    a0, a1 = T.instructions([lines[adds[0]]])[0][2], T.instructions([lines[adds[1]]])[0][2]
    lines[adds[0]] = f"\tv_add_f32_e32 {a0[0]}, {a0[1]}, {a1[1]}"
    lines[adds[1]] = f"\tv_add_f32_e32 {a1[0]}, {a0[2]}, {a1[2]}"
    sig = T.combine_tree_signature(lines)
    assert sig is not None and sig[0] == "((P0 + P2) + (P1 + P3))"   # read, and not the balanced tree


def test_planted_wave_tree_reorder_is_caught(reduce_asm):
    """Row shifts 1, 4, 2, 8 in place of 1, 2, 4, 8."""
    name, lines = next((n, list(l)) for n, l in T.kernels(reduce_asm).items() if "reduce_row_kernelIfLb1E" in n)
    lines = [l.replace("row_shr:2", "row_shr:@").replace("row_shr:4", "row_shr:2").replace("row_shr:@", "row_shr:4")
             for l in lines]
    sm, sq = T.leaf_chain(32, True)
    got = T.row_tree_signature(lines, False)
    assert got is not None and all("S8(S2(S4(S1(" in g for g in got)   # read, with the shifts reordered
    assert got != sorted([T.wave_tree(sm), T.wave_tree(sq)])


def test_planted_leaf_order_is_caught(reduce_asm):
    """Two elements of the leaf fold taken in the other order."""
    name, lines = next((n, list(l)) for n, l in T.kernels(reduce_asm).items() if "reduce_row_kernelIfLb1E" in n)
    adds = [k for k, l in enumerate(lines) if re.search(r"\bv_add_f32_e32\b", l)]
    # the chain's 3rd and 4th adds read x2 and x3: swap the elements they add
    i2, i3 = adds[1], adds[2]
    o2, o3 = T.instructions([lines[i2]])[0][2], T.instructions([lines[i3]])[0][2]
    lines[i2] = f"\tv_add_f32_e32 {o2[0]}, {o3[1] if o3[1] != o3[0] else o3[2]}, {o2[2] if o2[1] != o2[0] else o2[1]}"
    lines[i3] = f"\tv_add_f32_e32 {o3[0]}, {o2[1] if o2[1] != o2[0] else o2[2]}, {o3[2] if o3[1] != o3[0] else o3[1]}"
    sm, sq = T.leaf_chain(32, True)
    got = T.row_tree_signature(lines, False)
    assert got is not None and any("((e0 + e1) + e3) + e2)" in g for g in got)   # read, elements 2 and 3 swapped
    assert got != sorted([T.wave_tree(sm), T.wave_tree(sq)])
