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
        if "pipe_kernelILi320ELi256ELi2ELi4ELi4ELi1ELi0E" in name:
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
