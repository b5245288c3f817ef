"""Host-side walk of every global-to-LDS copy the pipelined GEMM kernels
issue (the bf16 pipe kernel, its two-tile-shape split kernel, and the W8A8
pipe kernel): for each compiled tile, on ragged shapes, every workgroup,
wave, lane, copy round and whole k tile, the 16 bytes read must lie inside
the operand's rows (a row past M or N reads the clamped last row) and inside
the split's k range, and the LDS bytes written inside the stage ring and
the kernel's LDS.

The walk restates the kernels' index arithmetic (copy slot s = r * waves +
wave, stage chunk c = 64 s + lane, A rows first, 16-byte chunk kc of a row
swizzled as kc ^ ((row >> 2) & 3) in 64-byte rows and kc ^ ((row >> 1) & 7)
in 128-byte rows, LDS byte (turn % stages * stage + 64 s + lane) * 16); the
two-stage tiles address a copy by a 32-bit byte offset from the tile's first
row, which must stay below 2^32.  The tile lists are read from the sources,
so a tile added there is walked too."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fixed_order_fp_amd", "csrc")


def _macro_rows(src, name):
    body = re.search(r"#define %s\(X\)(.*?)\n\n" % name, src, re.S).group(1)
    return [tuple(int(v) if v.strip().lstrip("-").isdigit() else v.strip() for v in m.split(","))
            for m in re.findall(r"X\(([^)]*)\)", body)]


def bf16_pipe_tiles():
    """(bm, bn, bk, wm, wn, ns) of the pipelined tiles, and the pairs as
    (bk, bm, bn, wm, wn, ns, bm2, bn2, wm2, wn2, ns2)."""
    src = open(os.path.join(CSRC, "bg_gemm_bf16.hip")).read()
    single = [(bm, bn, bk, wm, wn, ns) for i, bm, bn, bk, wm, wn, d, ns in _macro_rows(src, "BG_GEMM_TILES") if d == 2]
    dual = _macro_rows(src, "BG_GEMM_DUAL_TILES")
    return single, dual


def w8a8_pipe_tiles():
    """(bm, bn, wm, wn, ns, k tile bytes): two or three stages take 128-byte
    k tiles, rings of four or more 64-byte ones."""
    src = open(os.path.join(CSRC, "bg_w8a8.hip")).read()
    return [(bm, bn, wm, wn, ns, 128 if ns <= 3 else 64)
            for i, bm, bn, wm, wn, path, ns in _macro_rows(src, "BG_W8A8_TILES") if path == 2]


def walk(bm, bn, wm, wn, ns, M, N, ld_a, ld_b, k_begin, k_end, row_bytes, elt, out_lds, clamp=True):
    """Every copy of one tile shape over the whole grid of one split; returns
    (worst source overrun in bytes, worst k overrun in elements, the largest
    LDS byte written + 1)."""
    chunk = 16 // elt                       # elements per 16-byte chunk
    bk = row_bytes // elt                   # elements per k tile
    cpr = row_bytes // 16                   # chunks per tile row
    nw = wm * wn
    a_ch, b_ch = bm * cpr, bn * cpr
    stage = a_ch + b_ch
    slots = stage // 64
    rounds = -(-slots // nw)
    extra = slots % nw
    lds_bytes = max(ns * stage * 16, bm * bn * 2 if out_lds else 0)
    assert a_ch % 64 == 0 and b_ch % 64 == 0
    n_full = (k_end - k_begin) // bk
    tiles_m, tiles_n = -(-M // bm), -(-N // bn)
    wave = np.arange(nw)[:, None, None]
    lane = np.arange(64)[None, None, :]
    r = np.arange(rounds)[None, :, None]
    s = r * nw + wave
    issued = (r + 1 < rounds) | (extra == 0) | (s < slots)
    c = np.where(s < slots, s, 0) * 64 + lane
    is_a = c < a_ch
    row = np.where(is_a, c // cpr, (c - a_ch) // cpr)
    kc = (c % cpr) ^ (((row >> 2) & 3) if cpr == 4 else ((row >> 1) & 7))
    worst_src = worst_k = 0
    lds_hi = 0
    if n_full:
        turns = np.array([0, n_full - 1])  # the k offset grows with the turn: the ends bound it
        lds_off = ((turns[:, None, None, None] % ns) * stage + s[None] * 64 + lane[None]) * 16 + 16
        lds_hi = int(np.max(np.where(issued[None], lds_off, 0)))
    for tm in range(tiles_m):
        for tn in range(tiles_n):
            g = np.where(is_a, tm * bm + row, tn * bn + row)
            lim = np.where(is_a, M, N)
            if clamp:
                g = np.minimum(g, lim - 1)
            ld = np.where(is_a, ld_a, ld_b)
            size = np.where(is_a, M * ld_a, N * ld_b)
            if ns == 2:  # the byte offset from the tile's first row is 32-bit
                first_row = np.where(is_a, tm * bm, tn * bn)
                off = ((g - first_row) * ld + kc * chunk) * elt
                assert int(np.where(issued, off, 0).max()) + 16 <= 2 ** 32
            for t in ([0, n_full - 1] if n_full else []):
                k0 = k_begin + t * bk + kc * chunk
                first = g * ld + k0
                over_src = np.where(issued, (first + chunk) - size, -1)
                over_k = np.where(issued, (k0 + chunk) - k_end, -1)
                under = np.where(issued, first, 0)
                assert under.min() >= 0
                worst_src = max(worst_src, int(over_src.max()) * elt)
                worst_k = max(worst_k, int(over_k.max()))
    return worst_src, worst_k, lds_hi, lds_bytes


SHAPES = [(97, 136, 600), (256, 2560, 1024), (300, 504, 1000), (33, 70, 520), (4000, 200, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_pipe_copies_stay_in_bounds(M, N, K):
    single, dual = bf16_pipe_tiles()
    assert len(single) >= 20 and len(dual) >= 5
    assert {t[2] for t in single} == {32, 64} and {d[0] for d in dual} == {32, 64}
    shapes = set(single) | {(d[1], d[2], d[0]) + d[3:6] for d in dual} | {(d[6], d[7], d[0]) + d[8:] for d in dual}
    cuts = [0, (K // 3) // 8 * 8, K]  # two splits, the second deeper; and the whole range
    for bm, bn, bk, wm, wn, ns in sorted(shapes):
        for k0, k1 in ((0, K), (cuts[0], cuts[1]), (cuts[1], cuts[2])):
            src, kk, lds_hi, lds = walk(bm, bn, wm, wn, ns, M, N, K + 8, K, k0, k1, 2 * bk, 2, True)
            assert src <= 0 and kk <= 0, (bm, bn, bk, wm, wn, ns, M, N, K, k0, k1, src, kk)
            assert lds_hi <= lds <= 160 * 1024, (bm, bn, bk, ns, lds_hi, lds)


@pytest.mark.parametrize("M,N,K", [(128, 6144, 2048), (1024, 6144, 2048), (77, 200, 1040), (5, 64, 64)])
def test_w8a8_pipe_copies_stay_in_bounds(M, N, K):
    tiles = w8a8_pipe_tiles()
    assert len(tiles) >= 5 and {t[5] for t in tiles} == {64, 128}
    for bm, bn, wm, wn, ns, row_bytes in tiles:
        src, kk, lds_hi, lds = walk(bm, bn, wm, wn, ns, M, N, K, K, 0, K, row_bytes, 1, True)
        assert src <= 0 and kk <= 0, (bm, bn, wm, wn, ns, M, N, K, src, kk)
        assert lds_hi <= lds <= 160 * 1024


def test_a_planted_overrun_is_seen():
    """The walk has power: with the clamp of rows past M taken out it reports
    the read past the end of A."""
    bm, bn, wm, wn, ns = 128, 128, 2, 2, 4
    src, kk, _, _ = walk(bm, bn, wm, wn, ns, 100, 128, 1024, 1024, 0, 1024, 64, 2, True)
    assert src <= 0 and kk <= 0
    src, kk, _, _ = walk(bm, bn, wm, wn, ns, 100, 128, 1024, 1024, 0, 1024, 64, 2, True, clamp=False)
    assert src > 0
