"""GPU tests of the order-fixed bf16 GEMM through the C ABI.

Model-free checks first (exact integers, all-ones counts, schedule and
repeat invariance, batch invariance), then parity with the oracle under the
measured instruction model: 0 ULP on fp32 and bf16 outputs."""
import numpy as np
import pytest

import synth
from gpu_util import (from_dev_u16, oracle_desc, print_case, require_gpu, to_dev_u16)

pytestmark = pytest.mark.gpu

INSTRS = ["F32_32X32X16_BF16", "F32_16X16X32_BF16"]
SCHEDULES = {
    "F32_32X32X16_BF16": [dict(bm=320, bn=256, bk=64, waves_m=2, waves_n=4, load_path=2),
                          dict(bm=256, bn=320, bk=64, waves_m=4, waves_n=2, load_path=2, group_m=3),
                          dict(bm=192, bn=128, bk=64, waves_m=2, waves_n=2, load_path=2, stages=4),
                          dict(bm=128, bn=128, bk=64, waves_m=2, waves_n=2, load_path=2, stages=4),
                          dict(bm=128, bn=64, bk=64, waves_m=2, waves_n=2, load_path=2, stages=4),
                          dict(bm=64, bn=64, bk=64, waves_m=2, waves_n=2, load_path=2, stages=6),
                          dict(bm=32, bn=64, bk=64, waves_m=1, waves_n=2, load_path=2, stages=6),
                          dict(bm=320, bn=256, bk=32, waves_m=2, waves_n=4, load_path=2),
                          dict(bm=256, bn=320, bk=32, waves_m=4, waves_n=2, load_path=2),
                          dict(bm=256, bn=256, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=256, bn=256, bk=32, waves_m=2, waves_n=4, load_path=2, group_m=3),
                          dict(bm=256, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=192, bn=256, bk=32, waves_m=2, waves_n=4, load_path=2),
                          dict(bm=192, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=128, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=128, bn=64, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=64, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=64, bn=64, bk=32, waves_m=2, waves_n=2, load_path=2),
                          dict(bm=32, bn=128, bk=32, waves_m=1, waves_n=4, load_path=2),
                          dict(bm=32, bn=64, bk=32, waves_m=1, waves_n=2, load_path=2),
                          dict(bm=32, bn=32, bk=32, waves_m=1, waves_n=1, load_path=2, group_m=2),
                          dict(bm=32, bn=32, bk=32, waves_m=1, waves_n=1, load_path=2, stages=16),
                          dict(bm=64, bn=64, bk=32, waves_m=2, waves_n=2, load_path=2, stages=12),
                          dict(bm=128, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2, stages=8),
                          dict(bm=256, bn=256, bk=64, waves_m=2, waves_n=2, load_path=1),
                          dict(bm=256, bn=256, bk=64, waves_m=2, waves_n=4, load_path=1),
                          dict(bm=256, bn=128, bk=64, waves_m=2, waves_n=2, load_path=1),
                          dict(bm=128, bn=256, bk=64, waves_m=2, waves_n=2, load_path=1),
                          dict(bm=128, bn=128, bk=64, waves_m=2, waves_n=2, load_path=1, group_m=3),
                          dict(bm=128, bn=128, bk=64, waves_m=2, waves_n=2, load_path=0),
                          dict(bm=64, bn=64, bk=64, waves_m=2, waves_n=2),
                          dict(bm=32, bn=64, bk=64, waves_m=1, waves_n=2),
                          dict(bm=32, bn=32, bk=64, waves_m=1, waves_n=1)],
    "F32_16X16X32_BF16": [dict(bm=256, bn=256, bk=64, waves_m=2, waves_n=2, load_path=1),
                          dict(bm=256, bn=128, bk=64, waves_m=2, waves_n=2, load_path=1),
                          dict(bm=128, bn=128, bk=64, waves_m=2, waves_n=2),
                          dict(bm=64, bn=64, bk=64, waves_m=2, waves_n=2),
                          dict(bm=32, bn=32, bk=64, waves_m=1, waves_n=1),
                          dict(bm=16, bn=32, bk=64, waves_m=1, waves_n=2)],
}

# (other splits, last split) pairs: the last split, the cut rule's remainder,
# takes its own tile in the same launch (split_k > 1 only)
DUAL_SCHEDULES = [dict(bm=bm, bn=bn, bk=bk, waves_m=wm, waves_n=wn, load_path=2, stages=ns, last_bm=bm2,
                       last_bn=bn2, last_waves_m=wm2, last_waves_n=wn2, last_stages=ns2)
                  for bk, bm, bn, wm, wn, ns, bm2, bn2, wm2, wn2, ns2 in
                  [(32, 256, 256, 2, 2, 4, 64, 64, 2, 2, 8), (32, 256, 256, 2, 2, 4, 128, 64, 2, 2, 4),
                   (32, 256, 128, 2, 2, 4, 64, 64, 2, 2, 8), (32, 192, 128, 2, 2, 4, 64, 64, 2, 2, 8),
                   (32, 128, 128, 2, 2, 4, 64, 64, 2, 2, 8), (32, 256, 256, 2, 4, 4, 128, 64, 4, 2, 8),
                   (32, 256, 256, 2, 4, 4, 64, 128, 2, 4, 8), (64, 256, 256, 2, 4, 2, 128, 64, 4, 2, 4),
                   (64, 128, 128, 2, 2, 4, 64, 64, 2, 2, 6), (64, 128, 128, 2, 2, 4, 128, 64, 2, 2, 4)]]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_gemm(spec, A, B, out="fp32"):
    """A, B: numpy bf16 bits.  Returns numpy fp32 or bf16 bits."""
    import torch
    import fixed_order_fp_amd as bg
    d = bg.gemm_desc(spec, out_type=out)
    M, K = A.shape
    N = B.shape[0]
    dA, dB = to_dev_u16(A), to_dev_u16(B)
    dC = torch.empty((M, N), dtype=torch.float32 if out == "fp32" else torch.int16, device="cuda")
    nws = bg.gemm_workspace_bytes(d, M, N, K)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    bg.gemm_bf16(d, dA, dB, dC, ws)
    torch.cuda.synchronize()
    return dC.cpu().numpy() if out == "fp32" else from_dev_u16(dC)


# ---------------------------------------------------------------------------
# model-free
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("instr", INSTRS)
@pytest.mark.parametrize("K", [16, 24, 40, 136])
def test_small_integers_exact(instr, K):
    """Entries in {-4..4}: every order gives the exact integer (the K = 16
    small-integer workload, plus ragged K with a zero-padded short turn)."""
    print_case("small_int", instr, K)
    A, B = synth.gemm_small_int(K=K)
    for sched in SCHEDULES[instr]:
        C = run_gemm({"mfma": instr, "schedule": sched}, A, B)
        exact = synth.bf16_bits_to_f32(A).astype(np.int64) @ synth.bf16_bits_to_f32(B).astype(np.int64).T
        assert np.array_equal(C.astype(np.int64), exact), sched


@pytest.mark.parametrize("instr", INSTRS)
@pytest.mark.parametrize("K,S", [(512, 1), (512, 2), (9728, 1), (9728, 4), (9728, 16), (1000, 3), (16400, 64)])
def test_all_ones_count_every_k(instr, K, S):
    """All-ones operands: every output is exactly K for every split."""
    print_case("all_ones", instr, K, S)
    A = np.full((40, K), 0x3F80, dtype=np.uint16)
    B = np.full((72, K), 0x3F80, dtype=np.uint16)
    C = run_gemm({"mfma": instr, "split_k": S}, A, B)
    assert np.all(C == K)


@pytest.mark.parametrize("instr", INSTRS)
def test_schedules_do_not_move_bits(instr):
    """Every compiled tile shape and wave grid returns identical bytes
    ('Taming Bitwise Behavior' 3.2.2: BLOCK_M/N/K are speed knobs)."""
    print_case("schedules", instr)
    A = synth.bf16_spread(31, (97, 600), -20, 20)
    B = synth.bf16_spread(32, (136, 600), -20, 20)
    for S in (1, 2, 3):
        scheds = SCHEDULES[instr] + (DUAL_SCHEDULES if S > 1 and instr == "F32_32X32X16_BF16" else [])
        outs = [run_gemm({"mfma": instr, "split_k": S, "cut_unit": 64, "schedule": s}, A, B) for s in scheds]
        for s, o in zip(scheds[1:], outs[1:]):
            assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32)), (S, s)


@pytest.mark.parametrize("instr", INSTRS)
def test_repeats_are_identical(instr):
    print_case("repeats", instr)
    A, B = synth.gemm_small()
    first = run_gemm({"mfma": instr, "split_k": 2}, A, B)
    for _ in range(10):
        assert np.array_equal(run_gemm({"mfma": instr, "split_k": 2}, A, B).view(np.uint32),
                              first.view(np.uint32))


def test_rows_do_not_depend_on_batch_size():
    """Batch invariance on the batch-sweep recipe (reduced N): row i is the
    same for every M > i, with one descriptor for every M."""
    print_case("batch_invariance")
    X, W = synth.bf16_normal(1003, (512, 2560)), synth.bf16_normal(2003, (384, 2560), 0.0, 0.02)
    full = run_gemm({}, X, W, out="bf16")
    for M in (1, 8, 64, 300):
        assert np.array_equal(run_gemm({}, X[:M], W, out="bf16"), full[:M]), M


# ---------------------------------------------------------------------------
# parity with the oracle (needs the measured instruction model)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("instr", INSTRS)
@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_small_gemm_parity(instr, out):
    """The 32x64x512 workload, split-K = 2 cut at 256, partials combined as
    (p0 + p1); also S = 1 and 4; 0 ULP against the oracle."""
    import oracle
    A, B = synth.gemm_small()
    for S, cuts in ((2, [0, 256, 512]), (1, None), (4, None)):
        print_case("small_parity", instr, out, S)
        spec = {"mfma": instr, "split_k": S}
        if cuts:
            spec.update(cut_rule="EXPLICIT", cuts=cuts)
        if S == 4:
            spec["cut_unit"] = 64
        got = run_gemm(spec, A, B, out=out)
        ref = oracle.gemm_bf16(oracle_desc(dict(spec, out_type=out), instr), A, B)
        assert np.array_equal(got.view(np.uint16 if out == "bf16" else np.uint32),
                              ref.view(np.uint16 if out == "bf16" else np.uint32))


@pytest.mark.parametrize("instr", INSTRS)
def test_spread_parity_ragged(instr):
    """Exponent-spread inputs, ragged M, N, K spanning several tiles and a
    short last turn, S in {1, 3}: 0 ULP against the oracle."""
    import oracle
    A = synth.bf16_spread(41, (150, 712), -25, 25)
    B = synth.bf16_spread(42, (200, 712), -25, 25)  # N = 200: ldc a multiple of 8
    for S in (1, 3):
        spec = {"mfma": instr, "split_k": S, "cut_unit": 64}
        ref = oracle.gemm_bf16(oracle_desc(spec, instr), A, B)
        duals = DUAL_SCHEDULES if S > 1 and instr == "F32_32X32X16_BF16" else []
        for sched in [None] + SCHEDULES[instr] + duals:
            print_case("spread_parity", instr, S, sched)
            got = run_gemm(dict(spec, schedule=sched) if sched else spec, A, B)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), sched


def test_two_tile_shapes_on_tiny_outputs():
    """Every compiled (other splits, last split) pair on outputs much smaller
    than either tile (one row, eight columns; 33 x 40), the remainder split
    the deepest: 0 ULP against the oracle."""
    import oracle
    for M, N in ((1, 8), (33, 40)):
        A = synth.bf16_spread(90 + M, (M, 600), -20, 20)
        B = synth.bf16_spread(91 + N, (N, 600), -20, 20)
        spec = {"split_k": 3, "cut_unit": 64}
        ref = oracle.gemm_bf16(oracle_desc(dict(spec, out_type="fp32"), "F32_32X32X16_BF16"), A, B)
        for sched in DUAL_SCHEDULES:
            print_case("two tile shapes, tiny", M, N, sched)
            got = run_gemm(dict(spec, schedule=sched), A, B)
            assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (M, N, sched)


@pytest.mark.parametrize("S", [5, 6, 7, 9, 15])
def test_every_combine_width(S):
    """The combine kernels built for S = 5, 6 and 7 (an odd partial carried
    up at some level of the tree) and the runtime-S kernel (9, 15): exponent-
    spread operands, fp32 and bf16 output, 0 ULP against the oracle."""
    import oracle
    A = synth.bf16_spread(70 + S, (77, 1000), -20, 20)
    B = synth.bf16_spread(80 + S, (104, 1000), -20, 20)
    for out in ("fp32", "bf16"):
        print_case("combine width", S, out)
        spec = {"split_k": S, "cut_unit": 64}
        ref = oracle.gemm_bf16(oracle_desc(dict(spec, out_type=out), "F32_32X32X16_BF16"), A, B)
        got = run_gemm(spec, A, B, out=out)
        assert np.array_equal(got.view(np.uint16 if out == "bf16" else np.uint32),
                              ref.view(np.uint16 if out == "bf16" else np.uint32))


@pytest.mark.parametrize("instr", INSTRS)
def test_widest_split(instr):
    """S = 64, the most splits built: 63 spans of 256 and a last one of 272
    (K = 16400), exponent-spread operands, a six-level balanced combine;
    0 ULP against the oracle with fp32 and bf16 output."""
    import oracle
    A = synth.bf16_spread(61, (24, 16400), -20, 20)
    B = synth.bf16_spread(62, (40, 16400), -20, 20)
    for out in ("fp32", "bf16"):
        print_case("widest_split", instr, out)
        spec = {"mfma": instr, "split_k": 64}
        ref = oracle.gemm_bf16(oracle_desc(dict(spec, out_type=out), instr), A, B)
        got = run_gemm(spec, A, B, out=out)
        assert np.array_equal(got.view(np.uint16 if out == "bf16" else np.uint32),
                              ref.view(np.uint16 if out == "bf16" else np.uint32))


# ---------------------------------------------------------------------------
# the free-order twin (bench only): no bitwise contract, but it must compute
# the same product
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,split_k", [(1, 0), (8, 0), (64, 0), (200, 0), (64, 1), (64, 4)])
def test_free_twin_computes_the_product(M, split_k):
    import torch
    import fixed_order_fp_amd as bg
    X, W = synth.gemm_batch_sweep(M=M)
    W = W[:1024]
    N, K = W.shape
    print_case("free twin", M, N, K, split_k)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    bg.bench_gemm_bf16_free(to_dev_u16(X), to_dev_u16(W), dC, split_k)
    torch.cuda.synchronize()
    got = dC.cpu().numpy().astype(np.float64)
    a = synth.bf16_bits_to_f32(X).astype(np.float64)
    b = synth.bf16_bits_to_f32(W).astype(np.float64)
    exact = a @ b.T
    scale = np.abs(a) @ np.abs(b).T
    # fp32 accumulation over K terms plus at most 64 split partials
    assert np.all(np.abs(got - exact) <= (K / 8 + 64) * 2.0 ** -23 * scale + 1e-30)
    if split_k == 1:
        fixed = run_gemm({"mfma": "F32_32X32X16_BF16"}, X, W, out="fp32")
        assert np.array_equal(fixed.view(np.uint32), dC.cpu().numpy().view(np.uint32))


TILE_128_64DEEP = {"bm": 128, "bn": 128, "bk": 64, "waves_m": 2, "waves_n": 2, "load_path": 2, "stages": 4}


@pytest.mark.parametrize("M,N,K", [(1, 1024, 2560), (200, 1024, 2560), (333, 520, 1000), (130, 136, 328)])
def test_two_chain_twin_computes_the_product(M, N, K):
    """The two-chain free-order twin (bench only): the product within fp32
    accumulation error, over ragged tiles and a short last k tile, and on deep
    K other bits than the order-fixed kernel on the same tile -- its chains
    really are another order."""
    import torch
    import fixed_order_fp_amd as bg
    X, W = synth.gemm_batch_sweep(M=M)
    X = np.ascontiguousarray(X[:, :K])
    W = np.ascontiguousarray(W[:N, :K])
    print_case("two-chain twin", M, N, K)
    dC = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    bg.bench_gemm_bf16_two_chains(to_dev_u16(X), to_dev_u16(W), dC)
    torch.cuda.synchronize()
    got = dC.cpu().numpy()
    a = synth.bf16_bits_to_f32(X).astype(np.float64)
    b = synth.bf16_bits_to_f32(W).astype(np.float64)
    exact = a @ b.T
    scale = np.abs(a) @ np.abs(b).T
    assert np.all(np.abs(got.astype(np.float64) - exact) <= (K / 8 + 64) * 2.0 ** -23 * scale + 1e-30)
    fixed = run_gemm({"mfma": "F32_32X32X16_BF16", "schedule": TILE_128_64DEEP}, X, W, out="fp32")
    if K >= 1000:
        assert np.count_nonzero(fixed.view(np.uint32) != got.view(np.uint32)) > 0


# ---------------------------------------------------------------------------
# the full workloads, in the launch configuration the bench times (default
# schedules), on outputs sampled for the oracle
# ---------------------------------------------------------------------------
def test_batch_sweep_full_size():
    """N = 9728, K = 2560, bf16 out, M in {1, 8, 64, 512, 4000} with one
    descriptor: sampled outputs of every M match the oracle, and every row is
    bit-identical across all M (each M takes its own tile shape)."""
    import oracle
    X, W = synth.gemm_batch_sweep(M=4000)
    full = run_gemm({}, X, W, out="bf16")
    rng = np.random.default_rng(9)
    spec = oracle_desc({"out_type": "bf16"}, "F32_32X32X16_BF16")
    for M in (1, 8, 64, 512, 4000):
        print_case("batch sweep full size", M)
        C = full if M == 4000 else run_gemm({}, X[:M], W, out="bf16")
        assert np.array_equal(C, full[:M]), f"rows of M={M} differ from the same rows at M=4000"
        mi = rng.integers(0, M, 96)
        ni = rng.integers(0, W.shape[0], 96)
        ref = oracle.gemm_bf16_points(spec, X, W, mi, ni)
        assert np.array_equal(C[mi, ni], ref), f"M={M}: sampled outputs differ from the oracle"


@pytest.mark.parametrize("S", [1, 2, 4, 8, 16])
def test_splitk_sweep_full_size(S):
    """M = 256, N = 2560, K = 9728, fp32 out, cuts at multiples of 256 with
    the remainder last: sampled outputs match the oracle for each S."""
    import oracle
    A, B = synth.gemm_splitk_sweep()
    print_case("split-K sweep full size", S)
    C = run_gemm({"split_k": S}, A, B, out="fp32")
    rng = np.random.default_rng(100 + S)
    mi = rng.integers(0, A.shape[0], 96)
    ni = rng.integers(0, B.shape[0], 96)
    ref = oracle.gemm_bf16_points(oracle_desc({"split_k": S, "out_type": "fp32"}, "F32_32X32X16_BF16"), A, B, mi, ni)
    assert np.array_equal(C[mi, ni].view(np.uint32), ref.view(np.uint32))


@pytest.mark.slow
@pytest.mark.parametrize("S", [1, 2, 4, 8, 16])
def test_splitk_sweep_every_output(S):
    """M = 256, N = 2560, K = 9728 with the plan the bench times: all
    655,360 fp32 outputs of each S bit-identical to the oracle (about 12.7
    GFLOP of oracle work per S)."""
    import oracle
    A, B = synth.gemm_splitk_sweep()
    print_case("split-K sweep, every output", S)
    C = run_gemm({"split_k": S}, A, B, out="fp32")
    ref = oracle.gemm_bf16(oracle_desc({"split_k": S, "out_type": "fp32"}, "F32_32X32X16_BF16"), A, B)
    bad = np.flatnonzero(C.view(np.uint32) != ref.view(np.uint32))
    assert bad.size == 0, f"{bad.size} outputs differ, first at {np.unravel_index(bad[0], C.shape)}"


@pytest.mark.slow
def test_batch_sweep_row_bands_every_output():
    """M = 4000, N = 9728, K = 2560, bf16 out: eight bands of 32 rows spread
    over M (the first and the ragged last tile row included), every output
    of each band bit-identical to the oracle; the other M are shown
    row-identical to M = 4000 by test_batch_sweep_full_size."""
    import oracle
    X, W = synth.gemm_batch_sweep(M=4000)
    print_case("batch sweep M=4000, row bands")
    C = run_gemm({}, X, W, out="bf16")
    starts = [0, 320, 1000, 1630, 2240, 2880, 3500, 3968]
    rows = np.concatenate([np.arange(r, r + 32) for r in starts])
    ref = oracle.gemm_bf16(oracle_desc({"out_type": "bf16"}, "F32_32X32X16_BF16"), np.ascontiguousarray(X[rows]), W)
    bad = np.flatnonzero(C[rows] != ref)
    assert bad.size == 0, f"{bad.size} outputs differ, first at band row {np.unravel_index(bad[0], ref.shape)}"


def test_two_rounds_of_large_tiles_match_one_round_tiles():
    """More 320x256 tiles than CUs (3000 x 8000, 320 tiles in two rounds;
    ragged M, N and a short last k tile): bytes equal the 256x128 path, whose
    tiles fit one round, and sampled outputs match the oracle."""
    import oracle
    A = synth.bf16_spread(61, (3000, 1000), -20, 20)
    B = synth.bf16_spread(62, (8000, 1000), -20, 20)
    print_case("two rounds of 320x256 tiles, 3000x8000x1000")
    walk = run_gemm({"schedule": dict(bm=320, bn=256, bk=32, waves_m=2, waves_n=4, load_path=2)}, A, B, out="bf16")
    one = run_gemm({"schedule": dict(bm=256, bn=128, bk=32, waves_m=2, waves_n=2, load_path=2)}, A, B, out="bf16")
    assert np.array_equal(walk, one)
    # the same two rounds on 64-deep k tiles in two stages (1000 = 15 x 64 + 40: a short last tile)
    deep = run_gemm({"schedule": dict(bm=320, bn=256, bk=64, waves_m=2, waves_n=4, load_path=2)}, A, B, out="bf16")
    assert np.array_equal(deep, one)
    rng = np.random.default_rng(61)
    mi = rng.integers(0, 3000, 96)
    ni = rng.integers(0, 8000, 96)
    ref = oracle.gemm_bf16_points(oracle_desc({"out_type": "bf16"}, "F32_32X32X16_BF16"), A, B, mi, ni)
    assert np.array_equal(walk[mi, ni], ref)


@pytest.mark.parametrize("text", [
    '{"gemm": {"split_k": 2, "cut_rule": "EXPLICIT", "cuts": [0, 256, 512], "out_type": "fp32"}}',
    '{"gemm": {"split_k": 3, "cut_unit": 64, "out_type": "bf16"}}',
    '{"gemm": {"mfma": "F32_16X16X32_BF16", "split_k": 4, "cut_unit": 128, "out_type": "fp32", '
    '"schedule": {"bm": 64, "bn": 64, "bk": 64, "waves_m": 2, "waves_n": 2}}}',
    '{"gemm": {"split_k": 5, "cut_unit": 64, "out_type": "bf16", "schedule": {"bm": 128, "bn": 128, "bk": 32, '
    '"waves_m": 2, "waves_n": 2, "load_path": 2, "last_bm": 64, "last_bn": 64, "last_waves_m": 2, '
    '"last_waves_n": 2}}}',
])
def test_one_json_record_drives_both_sides(text):
    """[T] section 4: one frozen record.  The same descriptor text is read by
    the library (bg_desc_from_json) and by the oracle (its own reader); the
    outputs are bit-identical."""
    import torch
    import fixed_order_fp_amd as bg
    import oracle
    from gpu_util import profile
    print_case("json record", text)
    g, _ = bg.desc_from_json(text)
    spec, _ = oracle.desc_from_json(text, profile())
    A = synth.bf16_spread(71, (70, 512), -20, 20)
    B = synth.bf16_spread(72, (136, 512), -20, 20)
    out = spec["out_type"]
    dC = torch.empty((70, 136), dtype=torch.float32 if out == "fp32" else torch.int16, device="cuda")
    nws = bg.gemm_workspace_bytes(g, 70, 136, 512)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    bg.gemm_bf16(g, to_dev_u16(A), to_dev_u16(B), dC, ws)
    torch.cuda.synchronize()
    got = dC.cpu().numpy().view(np.uint32 if out == "fp32" else np.uint16)
    ref = oracle.gemm_bf16(spec, A, B)
    assert np.array_equal(got, ref.view(np.uint32 if out == "fp32" else np.uint16))


def test_64_deep_tiles_on_sliced_views():
    """The 64-deep tiles address their copies from each tile's first row by
    byte offsets that carry the leading dimension: operands that are column
    slices of wider buffers (lda, ldb > K), ragged M, N and K, every output
    against the oracle, for the two-stage tile and the four- and six-stage
    rings."""
    import torch
    import fixed_order_fp_amd as bg
    import oracle
    M, N, K = 700, 600, 1000
    A = synth.bf16_spread(71, (M, K), -20, 20)
    B = synth.bf16_spread(72, (N, K), -20, 20)
    ref = oracle.gemm_bf16(oracle_desc({"out_type": "bf16"}, "F32_32X32X16_BF16"), A, B)
    bufA = torch.zeros((M, K + 96), dtype=torch.int16, device="cuda")
    bufB = torch.zeros((N, K + 160), dtype=torch.int16, device="cuda")
    bufA[:, :K] = torch.from_numpy(A.view(np.int16)).cuda()
    bufB[:, :K] = torch.from_numpy(B.view(np.int16)).cuda()
    bufA[:, K:] = 0x7F80  # +inf past K: would show if a copy read beyond the row
    bufB[:, K:] = 0x7F80
    for sched in (dict(bm=320, bn=256, bk=64, waves_m=2, waves_n=4, load_path=2, stages=2),
                  dict(bm=256, bn=320, bk=64, waves_m=4, waves_n=2, load_path=2, stages=2),
                  dict(bm=192, bn=128, bk=64, waves_m=2, waves_n=2, load_path=2, stages=4),
                  dict(bm=64, bn=64, bk=64, waves_m=2, waves_n=2, load_path=2, stages=6),
                  dict(bm=32, bn=64, bk=64, waves_m=1, waves_n=2, load_path=2, stages=6)):
        print_case("64-deep tiles on sliced views", sched)
        d = bg.gemm_desc({"out_type": "bf16", "schedule": sched})
        dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
        bg.gemm_bf16(d, bufA[:, :K], bufB[:, :K], dC, None)
        torch.cuda.synchronize()
        got = dC.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), sched
