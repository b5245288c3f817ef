"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and its host-side descriptor logic (defaults, order
signature, cut rule, workspace size, refusals) behaves as documented."""
import ctypes as C
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitgemm.h")


@pytest.fixture(scope="module")
def bg():
    import fixed_order_fp_amd as bg
    if not os.path.exists(bg.LIB_PATH):
        from fixed_order_fp_amd import build
        build.build()
    bg.lib()
    return bg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bg_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported(bg):
    names = declared_functions()
    assert len(names) >= 15
    L = C.CDLL(bg.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # and the binding covers every one of them
    assert set(names) <= set(bg.exported_symbols())


def test_abi_version_and_profile(bg):
    assert bg.lib().bg_abi_version() == 2
    prof = bg.load_profile()
    from fixed_order_fp_amd.build import profile_hash
    assert bg.profile_hash() == profile_hash()
    assert prof["status"] == "measured"


def test_signature_covers_order_fields_only(bg):
    d1 = bg.gemm_desc({})
    d2 = bg.gemm_desc({"schedule": {"bm": 64, "bn": 64, "bk": 64, "waves_m": 2, "waves_n": 2}})
    assert bg.signature(d1) == bg.signature(d2)  # a speed knob moves no bit
    for change in ({"split_k": 2}, {"mfma": "F32_16X16X32_BF16"}, {"out_type": "fp32"},
                   {"cut_unit": 128}, {"mfma_profile_hash": 1}):
        assert bg.signature(bg.gemm_desc(change)) != bg.signature(d1), change
    r1, r2 = bg.reduce_desc({}), bg.reduce_desc({"schedule": {"leaves_per_wg": 8}})
    assert bg.signature(r1) == bg.signature(r2)
    assert bg.signature(bg.reduce_desc({"sq_fma": "unfused"})) != bg.signature(r1)


def test_cut_rule_and_workspace(bg):
    for S, spans in ((1, [9728]), (2, [4864, 4864]), (4, [2304] * 3 + [2816]),
                     (8, [1024] * 7 + [2560]), (16, [512] * 15 + [2048])):
        cuts = bg.split_cuts(bg.gemm_desc({"split_k": S}), 9728)
        assert [cuts[i + 1] - cuts[i] for i in range(S)] == spans
    assert bg.split_cuts(bg.gemm_desc({"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 256, 512]}),
                         512) == [0, 256, 512]
    assert bg.gemm_workspace_bytes(bg.gemm_desc({"split_k": 16}), 256, 2560, 9728) == 16 * 256 * 2560 * 4
    assert bg.gemm_workspace_bytes(bg.gemm_desc({}), 4000, 9728, 2560) == 0
    with pytest.raises(bg.BgError, match="BG_E_INVALID"):
        bg.split_cuts(bg.gemm_desc({"split_k": 2}), 256)  # an empty span


def _call_gemm(bg, d, M=32, N=64, K=512, lda=512, ptr=0x1000):
    return bg.lib().bg_gemm_bf16(C.byref(d), M, N, K, C.c_void_p(ptr), lda, C.c_void_p(ptr), K,
                                 C.c_void_p(ptr), N, None, 0, None)


def test_refusals_before_any_launch(bg):
    """Invalid or unsupported descriptors are refused synchronously, before the
    device is touched (the pointers here are never dereferenced)."""
    cases = [
        ({"split_k": 0}, 1),                     # BG_E_INVALID
        ({"version": 2}, 1),
        ({"acc_update": 1}, 2),                  # BG_E_UNSUPPORTED: separate add
        ({"short_turn": 1}, 2),                  # short turn first
        ({"k_slot_layout": 1}, 2),               # strided slots
        ({"combine": "SEQUENTIAL"}, 2),
        ({"partial_type": "bf16"}, 2),
        ({"mfma_profile_hash": 12345}, 6),       # BG_E_PROFILE
        ({"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 100, 512]}, 2),  # cut not a multiple of 8
        ({"split_k": 2}, 3),                     # BG_E_WORKSPACE: none given
        ({"schedule": {"bm": 48, "bn": 48, "bk": 64, "waves_m": 1, "waves_n": 1}}, 2),
    ]
    for spec, want in cases:
        st = _call_gemm(bg, bg.gemm_desc(spec))
        assert st == want, (spec, st, bg.lib().bg_last_error())
        assert bg.lib().bg_last_error()
    assert _call_gemm(bg, bg.gemm_desc({}), lda=513) == 4     # BG_E_ALIGN
    assert _call_gemm(bg, bg.gemm_desc({}), ptr=0x1004) == 4
    assert _call_gemm(bg, bg.gemm_desc({}), M=0) == 0          # nothing to do


def _call_w8a8(bg, d, M=64, N=64, K=256, lda=256, ldw=256, ldy=64, ptr=0x10000, acc=0):
    return bg.lib().bg_gemm_w8a8_pow2(C.byref(d), M, N, K, ptr, lda, ptr, ldw, ptr, ptr, ptr, ldy,
                                      acc or None, 64, None)


def test_w8a8_refusals_before_any_launch(bg):
    base = dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32", out_type="bf16",
                epilogue="W8A8_POW2")
    cases = [
        (dict(base, mfma="F32_32X32X16_BF16"), {}, 1),
        (dict(base, epilogue="NONE"), {}, 1),
        (dict(base, acc_type="fp32"), {}, 1),
        (dict(base, a_type="bf16"), {}, 1),
        (dict(base, split_k=2), {}, 2),
        (dict(base, schedule=dict(bm=96, bn=96, waves_m=2, waves_n=2)), {}, 2),
        (base, dict(K=131072, lda=131072, ldw=131072), 2),   # beyond the exact int32 range
        (base, dict(K=0), 1),
        (base, dict(lda=100), 1),                            # lda < K
        (base, dict(lda=264), 4),                            # not a multiple of 16
        (base, dict(ldy=68), 4),                             # not a multiple of 8
        (base, dict(ptr=0x10008), 4),
        (base, dict(M=0), 0),
    ]
    for spec, args, want in cases:
        st = _call_w8a8(bg, bg.gemm_desc(spec), **args)
        assert st == want, (spec, args, st, bg.lib().bg_last_error())


def test_shapes_past_one_launch_are_refused(bg):
    """A dispatch counts each grid dimension's work-items in 32 bits: shapes
    whose grid would pass that are refused with BG_E_UNSUPPORTED before any
    launch (and before the pointers, never dereferenced here, are used); the
    largest shapes that fit are not refused on that ground."""
    L, p, big = bg.lib(), C.c_void_p(0x10000), C.c_size_t(1 << 62)
    unsup = 2
    # bf16 GEMM: 2^20 x 2^20 outputs in 320 x 256 tiles of 512 lanes
    assert _call_gemm(bg, bg.gemm_desc({}), M=1 << 20, N=1 << 20, K=512) == unsup
    # W8A8: the same outputs in 128 x 192 tiles
    d8 = bg.gemm_desc(dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32",
                           out_type="bf16", epilogue="W8A8_POW2"))
    assert _call_w8a8(bg, d8, M=1 << 20, N=1 << 20, ldy=1 << 20) == unsup
    # reductions: a workgroup per row (2^24 rows), and the one-pass column path
    # (2^27 fp32 columns at 64 lanes each)
    row, col = bg.reduce_desc({"axis": "row"}), bg.reduce_desc({"axis": "col", "in_type": "fp32"})
    full = bg.reduce_desc({"axis": "col", "in_type": "fp32", "schedule": {"leaves_per_wg": 256}})
    red = lambda d, rows, cols: L.bg_reduce_tree(C.byref(d), rows, cols, p, cols, p, p, p, big, None)
    assert red(row, 1 << 24, 8) == unsup
    assert red(full, 32, 1 << 27) == unsup
    assert red(col, 64, 1 << 32) == unsup
    # int8 steps: a workgroup per row, per two rows
    assert L.bg_quantize_act_int8(1 << 24, 16, p, 16, p, 16, p, None) == unsup
    assert L.bg_requantize_weights_pow2((1 << 25) - 1, 16, p, 16, p, 0, C.c_void_p(1 << 40), 16, p, None) == unsup
    # Ozaki: M below 2^24 (slicing) and M x N below 2^32 (combine)
    oz = lambda M, N: L.bg_gemm_ozaki(M, N, 64, 0, p, 64, p, 64, 0, p, N, p, big, None)
    assert oz(1 << 24, 8) == unsup
    assert oz(1 << 16, 1 << 16) == unsup
    size = C.c_size_t()
    assert L.bg_gemm_ozaki_workspace_bytes(1 << 30, 1 << 30, 64, C.byref(size)) == unsup
    assert L.bg_gemm_ozaki_workspace_bytes(1 << 12, 1 << 12, 64, C.byref(size)) == 0
    assert L.bg_gemm_workspace_bytes(C.byref(bg.gemm_desc({"split_k": 2})), 1 << 40, 1 << 40, 512,
                                     C.byref(size)) == unsup
    # the longest row (64 blocks of 8192) and column (64 blocks of 32 leaves of 32) built
    assert red(row, 2, 64 * 8192 + 1) == unsup
    assert red(col, 64 * 32 * 32 + 1, 40) == unsup
    assert b"65,536 rows" in L.bg_last_error()
    # the GEMM with a fused reduction: at most 1024 leaves on the reduced axis
    dg = bg.gemm_desc({}, out_type="bf16")
    fused = lambda axis, M, N: L.bg_gemm_bf16_reduce(C.byref(dg), C.byref(bg.reduce_desc({"in_type": "fp32",
                                                     "axis": axis})), M, N, 64, p, 64, p, 64, p,
                                                     (N + 7) // 8 * 8, p, p, p, big, None)
    assert fused("col", 32769, 40) == unsup and fused("row", 3, 32769) == unsup
    # the probe: 64 lanes per case
    assert L.bg_probe_mfma(0, 1 << 26, p, p, p, p, None) == unsup


def test_fused_reduce_refuses_k_off_the_chunk_grid(bg):
    """K is the split's end, a cut point: like bg_gemm_bf16 the fused call takes
    it only on the 8-element chunk grid, even where lda leaves room for the
    chunk (a sliced view K = 20 of rows of 24): refused before any launch."""
    L, p, big = bg.lib(), C.c_void_p(0x10000), C.c_size_t(1 << 40)
    dg = bg.gemm_desc({}, out_type="fp32")
    rd = bg.reduce_desc({"in_type": "fp32", "axis": "col"})
    call = lambda K, ld: L.bg_gemm_bf16_reduce(C.byref(dg), C.byref(rd), 64, 64, K, p, ld, p, ld, p, 64,
                                               p, p, p, big, None)
    assert call(20, 24) == 2
    assert b"multiple of 8" in L.bg_last_error()
    assert _call_gemm(bg, bg.gemm_desc({}), K=20, lda=24) == 2   # the plain GEMM alike


# ---------------------------------------------------------------------------
# descriptors as JSON text
# ---------------------------------------------------------------------------
def _struct_bytes(d):
    return bytes(memoryview(d))


JSON_DOCS = [
    '{"gemm": {}}',
    '{"gemm": {"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 256, 512], "out_type": "fp32"}}',
    '{"gemm": {"split_k": 16, "out_type": "fp32", "schedule": {"bm": 128, "bn": 64, "bk": 32, '
    '"waves_m": 2, "waves_n": 2, "load_path": 2, "stages": 8}}}',
    '{"gemm": {"split_k": 16, "out_type": "fp32", "schedule": {"bm": 256, "bn": 256, "bk": 32, "waves_m": 2, '
    '"waves_n": 4, "load_path": 2, "stages": 4, "last_bm": 128, "last_bn": 64, "last_waves_m": 4, '
    '"last_waves_n": 2, "last_stages": 8}}}',
    '{"gemm": {"mfma": "F32_16X16X32_BF16", "combine": "SEQUENTIAL", "cut_unit": 128, "split_k": 3}}',
    '{"gemm": {"mfma": "I32_32X32X32_I8", "a_type": "int8", "b_type": "int8", "acc_type": "int32", '
    '"out_type": "bf16", "epilogue": "W8A8_POW2"}}',
    '{"reduce": {"axis": "col", "in_type": "bf16", "op": "sum", "sq_fma": "unfused", '
    '"schedule": {"leaves_per_wg": 8}}}',
    '{"gemm": {"acc_update": "SEPARATE_ADD", "short_turn": "FIRST", "k_slot_layout": "STRIDED"}, '
    '"reduce": {"op": "sumsq"}}',
]


@pytest.mark.parametrize("text", JSON_DOCS)
def test_json_round_trip_keeps_the_record(bg, text):
    """[T] section 4: the descriptor is a frozen record.  Text read by the
    library, written back and read again gives the same bytes (order fields
    and schedule) and the same signature."""
    g1, r1 = bg.desc_from_json(text)
    back = bg.desc_to_json(g1, r1)
    g2, r2 = bg.desc_from_json(back)
    assert _struct_bytes(g1) == _struct_bytes(g2) and _struct_bytes(r1) == _struct_bytes(r2)
    assert bg.signature(g1) == bg.signature(g2) and bg.signature(r1) == bg.signature(r2)
    assert bg.desc_to_json(g2, r2) == back          # the writer is canonical


def test_json_agrees_with_field_by_field_construction(bg):
    spec = {"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 256, 512], "out_type": "fp32"}
    g, _ = bg.desc_from_json('{"gemm": %s}' % __import__("json").dumps(spec))
    d = bg.gemm_desc(spec)
    assert bg.signature(g) == bg.signature(d) and _struct_bytes(g) == _struct_bytes(d)
    # an absent member leaves the defaults, including the library's profile hash
    g0, r0 = bg.desc_from_json("{}")
    assert _struct_bytes(g0) == _struct_bytes(bg.gemm_desc({}))
    assert _struct_bytes(r0) == _struct_bytes(bg.reduce_desc({}))
    assert g0.mfma_profile_hash == bg.profile_hash()
    # the hash is part of the record: another profile is another signature
    g1, _ = bg.desc_from_json('{"gemm": {"mfma_profile_hash": "0x0000000000000001"}}')
    assert g1.mfma_profile_hash == 1 and bg.signature(g1) != bg.signature(g0)


@pytest.mark.parametrize("text, why", [
    ('{"gemm": {"split_k": 2,}}', "malformed"),
    ('{"gemm": {"split_k": 2}', "malformed"),
    ('{"gemm": {"split_k": 2}} x', "after the document"),
    ('[1, 2]', "must be an object"),
    ('{"gemm": {"splitk": 2}}', "unknown gemm key"),
    ('{"gemm": {"split_k": "2"}}', "must be an integer"),
    ('{"gemm": {"split_k": 2.0}}', "integers"),
    ('{"gemm": {"split_k": -1}}', "must be an integer"),
    ('{"gemm": {"mfma": "F32_32X32X8_BF16"}}', "unknown value"),
    ('{"gemm": {"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 512]}}', "split_k + 1"),
    ('{"gemm": {"cuts": [0, "256"]}}', "array of integers"),
    ('{"gemm": {"mfma_profile_hash": 123}}', "hex"),
    ('{"gemm": {"mfma_profile_hash": "0x12345"}}', "hex"),
    ('{"gemm": {"split_k": 2, "split_k": 4}}', "duplicate"),
    ('{"gemm": {"schedule": {"tile": 3}}}', "unknown gemm schedule key"),
    ('{"reduce": {"axis": "diagonal"}}', "unknown value"),
    ('{"gemm": {}, "profile": {}}', "unknown top-level key"),
    ('', "malformed"),
])
def test_json_refusals(bg, text, why):
    """A document that is not exactly a descriptor record is refused with
    BG_E_INVALID, and the output structs are left as they were."""
    L = bg.lib()
    g, r = bg.gemm_desc({"split_k": 5}), bg.reduce_desc({"axis": "col"})
    before = (_struct_bytes(g), _struct_bytes(r))
    st = L.bg_desc_from_json(text.encode(), C.byref(g), C.byref(r))
    assert st == 1, (text, st)
    assert why.encode() in L.bg_last_error(), L.bg_last_error()
    assert (_struct_bytes(g), _struct_bytes(r)) == before


def test_json_writer_buffer_and_names(bg):
    L = bg.lib()
    g = bg.gemm_desc({})
    n = C.c_size_t(0)
    assert L.bg_desc_to_json(C.byref(g), None, None, 0, C.byref(n)) == 1 and n.value > 100
    small = C.create_string_buffer(n.value)          # one byte short of the NUL
    assert L.bg_desc_to_json(C.byref(g), None, small, n.value, C.byref(n)) == 1
    assert b"buffer too small" in L.bg_last_error()
    g.mfma = 99                                      # a value with no name
    big = C.create_string_buffer(4096)
    assert L.bg_desc_to_json(C.byref(g), None, big, 4096, C.byref(n)) == 1
    assert L.bg_desc_to_json(None, None, big, 4096, C.byref(n)) == 1
    assert L.bg_desc_from_json(None, C.byref(g), None) == 1


# ---------------------------------------------------------------------------
# the plan query: which tiles a call would launch (host only)
# ---------------------------------------------------------------------------
def test_plan_reports_the_schedule_and_the_choice(bg):
    """An explicit schedule comes back as given (stage counts filled in); the
    library's choice is a compiled tile; a split sweep whose remainder split
    is four times deeper than the others (256 x 2560 x 9728, S = 16: fifteen
    spans of 512 and one of 2048) gives that split its own smaller tile."""
    sched = dict(bm=128, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2, stages=8)
    got = bg.gemm_bf16_plan(bg.gemm_desc({"split_k": 2, "schedule": sched}), 300, 500, 1024)
    assert {k: got[k] for k in sched} == sched and got["last_bm"] == 0
    pair = dict(sched, stages=0, last_bm=64, last_bn=64, last_waves_m=2, last_waves_n=2)
    got = bg.gemm_bf16_plan(bg.gemm_desc({"split_k": 3, "schedule": pair}), 300, 500, 1024)
    assert (got["stages"], got["last_bm"], got["last_bn"], got["last_stages"]) == (4, 64, 64, 8)
    one = bg.gemm_bf16_plan(bg.gemm_desc({"out_type": "bf16"}), 4000, 9728, 2560)
    assert (one["bm"], one["bn"], one["last_bm"]) == (320, 256, 0)
    deep = bg.gemm_bf16_plan(bg.gemm_desc({"split_k": 16, "out_type": "fp32"}), 256, 2560, 9728)
    assert deep["last_bm"] and deep["last_bm"] * deep["last_bn"] < deep["bm"] * deep["bn"]
    assert deep["last_waves_m"] * deep["last_waves_n"] == deep["waves_m"] * deep["waves_n"]
    for S in (1, 2, 4, 8, 16):  # every choice is launchable: the plan fed back is accepted as given
        d = bg.gemm_desc({"split_k": S, "out_type": "fp32"})
        p = bg.gemm_bf16_plan(d, 256, 2560, 9728)
        assert bg.gemm_bf16_plan(bg.gemm_desc({"split_k": S, "out_type": "fp32", "schedule": p}),
                                 256, 2560, 9728) == p


@pytest.mark.parametrize("S,sched,why", [
    (1, dict(bm=256, bn=256, bk=32, waves_m=2, waves_n=4, load_path=2, last_bm=128, last_bn=64, last_waves_m=4,
             last_waves_n=2), "split_k > 1"),
    (4, dict(last_bm=64, last_bn=64, last_waves_m=2, last_waves_n=2), "other splits' tile"),
    (4, dict(bm=256, bn=256, bk=32, waves_m=2, waves_n=2, load_path=2, last_bm=32, last_bn=32, last_waves_m=1,
             last_waves_n=1), "not compiled"),
    (4, dict(bm=256, bn=256, bk=32, waves_m=2, waves_n=4, load_path=2, last_bm=64, last_bn=64, last_waves_m=2,
             last_waves_n=2), "not compiled"),
    (4, dict(bm=128, bn=128, bk=64, waves_m=2, waves_n=2, load_path=1, last_bm=64, last_bn=64, last_waves_m=2,
             last_waves_n=2), "not compiled"),
])
def test_last_split_tile_refusals(bg, S, sched, why):
    """A last-split tile needs a split, the other splits' tile, and a
    compiled pair with the same number of waves; the plan query and the call
    refuse alike, before any launch."""
    d = bg.gemm_desc({"split_k": S, "schedule": sched})
    with pytest.raises(bg.BgError) as e:
        bg.gemm_bf16_plan(d, 300, 504, 1024)
    assert e.value.status == "BG_E_UNSUPPORTED" and why in str(e.value)
    p = 0x10000  # never dereferenced
    st = bg.lib().bg_gemm_bf16(C.byref(d), 300, 504, 1024, p, 1024, p, 1024, p, 504, p, 1 << 30, None)
    assert st == 2 and why in bg.lib().bg_last_error().decode()


def test_every_planned_schedule_is_compiled(bg):
    """Across shapes and split counts (deep remainder splits among them) the
    library's choice is always a compiled tile or pair: fed back as an
    explicit schedule it is accepted and planned identically."""
    n = 0
    for M in (1, 8, 32, 64, 65, 100, 256, 300, 1000, 4000):
        for N in (64, 500, 2560, 9728):
            for K in (2048, 9728, 20000):
                for S in (1, 2, 3, 4, 5, 8, 16, 32):
                    if 256 * S > K:
                        continue
                    spec = {"split_k": S, "out_type": "fp32"}
                    p = bg.gemm_bf16_plan(bg.gemm_desc(spec), M, N, K)
                    assert bg.gemm_bf16_plan(bg.gemm_desc(dict(spec, schedule=p)), M, N, K) == p, (M, N, K, S, p)
                    n += p["last_bm"] > 0
    assert n > 0  # some of them take a pair of tiles


def test_two_chain_twin_refusals(bg):
    """The two-chain free-order twin keeps bg_gemm_bf16's argument rules and
    refuses before any launch (the pointers are never dereferenced)."""
    p = 0x10000
    f = bg.lib().bg_bench_gemm_bf16_two_chains
    assert f(64, 64, 0, p, 64, p, 64, p, 64, None) == 1             # K < 1
    assert f(64, 64, 256, p, 128, p, 256, p, 64, None) == 1         # lda < K
    assert f(64, 64, 100, p, 104, p, 104, p, 64, None) == 2         # K off the multiple-of-8 grid
    assert f(64, 64, 256, p + 4, 256, p, 256, p, 64, None) == 4     # misaligned
    assert f(64, 64, 256, p, 20_000_000, p, 256, p, 64, None) == 2  # 127 x 2e7 x 2 bytes > 2^32
    assert "32-bit copy offsets" in bg.lib().bg_last_error().decode()
    assert f(0, 64, 256, p, 256, p, 256, p, 64, None) == 0          # nothing to do


def test_copy_offset_limit(bg):
    """The 64-deep two-stage tiles address their copies by 32-bit byte
    offsets from the tile's first row: an explicit schedule whose
    (bm - 1) x lda x 2 bytes reaches 2^32 is refused before any launch
    (bf16, and the W8A8 two-stage tiles with one byte per element), and the
    library's own choice falls back to the 32-deep ring there."""
    p = 0x10000  # never dereferenced
    big = 7_000_000  # 319 x 7e6 x 2 bytes > 2^32; a multiple of 16
    d = bg.gemm_desc({"schedule": {"bm": 320, "bn": 256, "bk": 64, "waves_m": 2, "waves_n": 4, "load_path": 2,
                                   "stages": 2}})
    st = bg.lib().bg_gemm_bf16(C.byref(d), 4000, 9728, 2560, p, big, p, 2560, p, 9728, None, 0, None)
    assert st == 2 and "32-bit offsets" in bg.lib().bg_last_error().decode()
    st = bg.lib().bg_gemm_bf16(C.byref(d), 4000, 9728, 2560, p, 2560, p, 9_000_000, p, 9728, None, 0, None)
    assert st == 2 and "32-bit offsets" in bg.lib().bg_last_error().decode()  # 255 x 9e6 x 2 > 2^32
    # the chooser: contiguous operands of a huge K take the 32-deep tile, of
    # the headline's K the 64-deep one
    free = bg.gemm_desc({"out_type": "bf16"})
    assert bg.gemm_bf16_plan(free, 4000, 9728, big)["bk"] == 32
    assert bg.gemm_bf16_plan(free, 4000, 9728, 2560)["bk"] == 64
    w = bg.gemm_desc(dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32", out_type="bf16",
                          epilogue="W8A8_POW2", schedule={"bm": 256, "bn": 256, "waves_m": 2, "waves_n": 4,
                                                          "load_path": 2, "stages": 2}))
    huge = 20_000_000  # 255 x 2e7 bytes > 2^32
    st = bg.lib().bg_gemm_w8a8_pow2(C.byref(w), 1024, 1024, 2048, p, huge, p, 2048, p, p, p, 1024, None, 0, None)
    assert st == 2 and "32-bit offsets" in bg.lib().bg_last_error().decode()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: any other --gpus exits with status 2 and a
    message, before anything touches a device."""
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "measures one GPU" in r.stderr
