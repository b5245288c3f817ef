"""GPU tests of the GEMM with fused reductions of C (bg_gemm_bf16_reduce)
through the C ABI.  The reference is the oracle's own composition: the fp32 C
of the same descriptor (oracle.gemm_bf16 / gemm_bf16_points), then the
oracle's fixed-order reduction of it along the requested axis.  The C the
call writes must equal bg_gemm_bf16's bit for bit, and the reductions must not
depend on the tile."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import from_dev_u16, oracle_desc, print_case, require_gpu, to_dev_u16

pytestmark = pytest.mark.gpu

# the tiles built with the fused reductions (bm, bn, waves_m, waves_n, stages)
RED_TILES = [(320, 256, 2, 4, 4), (256, 128, 2, 2, 4), (64, 64, 2, 2, 8)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def same(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def run(A, B, axis, op="sum_and_sumsq", fused=True, out="bf16", tile=None):
    """A, B: bf16 bits.  Returns (C numpy, sum, sumsq) from bg_gemm_bf16_reduce."""
    import torch
    import fixed_order_fp_amd as bg
    M, K = A.shape
    N = B.shape[0]
    sched = {} if tile is None else dict(bm=tile[0], bn=tile[1], bk=32, waves_m=tile[2], waves_n=tile[3],
                                         load_path=2, stages=tile[4])
    d = bg.gemm_desc({"mfma": "F32_32X32X16_BF16", "schedule": sched}, out_type=out)
    rd = bg.reduce_desc({"in_type": "fp32", "axis": axis, "op": op, "sq_fma": "fused" if fused else "unfused"})
    dA, dB = to_dev_u16(A), to_dev_u16(B)
    ldc = (N + 7) // 8 * 8  # leading dimensions are multiples of 8
    dC = torch.empty((M, ldc), dtype=torch.float32 if out == "fp32" else torch.int16, device="cuda")[:, :N]
    n_out = N if axis == "col" else M
    s = torch.full((n_out + 1,), float("nan"), dtype=torch.float32, device="cuda")
    q = torch.full((n_out + 1,), float("nan"), dtype=torch.float32, device="cuda")
    nws = bg.gemm_bf16_reduce_workspace_bytes(d, rd, M, N, K)
    ws = torch.empty(max(nws, 4) // 4, dtype=torch.float32, device="cuda")
    bg.gemm_bf16_reduce(d, rd, dA, dB, dC, s[:n_out], q[:n_out], ws)
    torch.cuda.synchronize()
    s, q = s.cpu().numpy(), q.cpu().numpy()
    assert np.isnan(s[n_out]) and np.isnan(q[n_out]), "wrote past the last output"
    C = dC.cpu().numpy() if out == "fp32" else from_dev_u16(dC.contiguous())
    return C, s[:n_out], q[:n_out]


def oracle_ref(A, B, axis, fused=True):
    spec = oracle_desc({"mfma": "F32_32X32X16_BF16", "out_type": "fp32"})
    C32 = oracle.gemm_bf16(spec, A, B)
    return C32, oracle.reduce(C32, axis, leaf_len=32, sq_fused=fused, in_type="fp32")


@pytest.mark.parametrize("axis", ["col", "row"])
@pytest.mark.parametrize("M,N,K", [(300, 500, 256), (64, 128, 64), (33, 65, 16), (40, 300, 128),
                                   (700, 1000, 512), (1, 96, 48)])
def test_against_oracle_composition(axis, M, N, K):
    """Ragged M and N (short last leaves, partial tiles), short K, M <= 64."""
    print_case("gemm_reduce", axis, M, N, K)
    A = synth.bf16_normal(500 + M, (M, K))
    B = synth.bf16_normal(600 + N, (N, K), sigma=0.05)
    C32, (rs, rq) = oracle_ref(A, B, axis)
    C, s, q = run(A, B, axis, out="fp32")
    assert same(C, C32), "C differs from the oracle"
    assert same(s, rs) and same(q, rq)


@pytest.mark.parametrize("axis,M,N", [("col", 32768, 40), ("col", 32761, 40), ("row", 3, 32768),
                                     ("row", 3, 32763)])
def test_longest_reduced_axis(axis, M, N):
    """The longest reduced axis built: 1024 leaves (a full 32-leaf run per
    wave of the second kernel), and the same with a short last leaf."""
    print_case("gemm_reduce longest", axis, M, N)
    A = synth.bf16_normal(701, (M, 64))
    B = synth.bf16_normal(702, (N, 64), sigma=0.05)
    C32, (rs, rq) = oracle_ref(A, B, axis)
    C, s, q = run(A, B, axis, out="fp32")
    assert same(C, C32), "C differs from the oracle"
    assert same(s, rs) and same(q, rq)


@pytest.mark.parametrize("axis", ["col", "row"])
def test_every_tile_and_the_output_types(axis):
    """Each tile built with the reductions gives the same reductions; the bf16
    C equals bg_gemm_bf16's; unfused squares and single ops."""
    import torch
    import fixed_order_fp_amd as bg
    print_case("gemm_reduce tiles", axis)
    M, N, K = 520, 704, 320
    A = synth.bf16_normal(71, (M, K))
    B = synth.bf16_normal(72, (N, K), sigma=0.05)
    C32, (rs, rq) = oracle_ref(A, B, axis)
    _, (us, uq) = oracle_ref(A, B, axis, fused=False)
    d = bg.gemm_desc({"mfma": "F32_32X32X16_BF16"}, out_type="bf16")
    dC = torch.empty((M, N), dtype=torch.int16, device="cuda")
    bg.gemm_bf16(d, to_dev_u16(A), to_dev_u16(B), dC, None)
    torch.cuda.synchronize()
    Cb = from_dev_u16(dC)
    for tile in RED_TILES:
        C, s, q = run(A, B, axis, out="bf16", tile=tile)
        assert np.array_equal(C, Cb), tile
        assert same(s, rs) and same(q, rq), tile
        _, s, q = run(A, B, axis, fused=False, tile=tile)
        assert same(s, us) and same(q, uq), tile
    _, s, q = run(A, B, axis, op="sum")
    assert same(s, rs) and np.isnan(q).all()
    _, s, q = run(A, B, axis, op="sumsq")
    assert same(q, rq) and np.isnan(s).all()


@pytest.mark.parametrize("axis", ["col", "row"])
def test_headline_shape_sampled(axis):
    """M=4000, N=9728, K=2560 (the batch-sweep weights): sampled columns (or
    rows) of C computed by the oracle in full along the reduced axis."""
    print_case("gemm_reduce headline", axis)
    X, W = synth.gemm_batch_sweep(M=4000)
    C, s, q = run(X, W, axis, out="bf16")
    rng = np.random.default_rng(3)
    spec = oracle_desc({"mfma": "F32_32X32X16_BF16", "out_type": "fp32"})
    if axis == "col":
        cols = np.sort(rng.choice(9728, 6, replace=False))
        mi = np.repeat(np.arange(4000), len(cols))
        ni = np.tile(cols, 4000)
        sub = oracle.gemm_bf16_points(spec, X, W, mi, ni).reshape(4000, len(cols))
        rs, rq = oracle.reduce(sub, "col", leaf_len=32, in_type="fp32")
        assert same(s[cols], rs) and same(q[cols], rq)
    else:
        rows = np.sort(rng.choice(4000, 3, replace=False))
        mi = np.repeat(rows, 9728)
        ni = np.tile(np.arange(9728), len(rows))
        sub = oracle.gemm_bf16_points(spec, X, W, mi, ni).reshape(len(rows), 9728)
        rs, rq = oracle.reduce(sub, "row", leaf_len=32, in_type="fp32")
        assert same(s[rows], rs) and same(q[rows], rq)


def test_argument_errors():
    import torch
    import fixed_order_fp_amd as bg
    A = torch.zeros((64, 64), dtype=torch.int16, device="cuda")
    Cc = torch.zeros((64, 64), dtype=torch.float32, device="cuda")
    s = torch.zeros(64, dtype=torch.float32, device="cuda")
    ws = torch.zeros(1 << 16, dtype=torch.float32, device="cuda")
    ok_rd = bg.reduce_desc({"in_type": "fp32", "axis": "col", "op": "sum"})
    with pytest.raises(bg.BgError):
        bg.gemm_bf16_reduce(bg.gemm_desc({"split_k": 2}, out_type="fp32"), ok_rd, A, A, Cc, s, None, ws)
    with pytest.raises(bg.BgError):
        bg.gemm_bf16_reduce(bg.gemm_desc({}, out_type="fp32"), bg.reduce_desc({"in_type": "bf16", "axis": "col"}),
                            A, A, Cc, s, None, ws)
    with pytest.raises(bg.BgError):  # workspace too small
        bg.gemm_bf16_reduce(bg.gemm_desc({}, out_type="fp32"), ok_rd, A, A, Cc, s, None, ws[:1])
    big = bg.reduce_desc({"in_type": "fp32", "axis": "row", "op": "sum"})
    assert bg.gemm_bf16_reduce_workspace_bytes(bg.gemm_desc({}), big, 4, 40000, 64) == 1250 * 4 * 4


@pytest.mark.parametrize("axis", ["col", "row"])
def test_sliced_operand_views(axis):
    """A and B given as views of wider rows (K = 24 of rows of 40, a k range
    that is not a whole 32-deep tile), with a short last leaf: the padding
    columns past K hold large values that must not enter any product, and
    the fused GEMM and the plain GEMM agree with the oracle on the sliced
    operands.  (K not a multiple of 8 is refused: test_abi.)"""
    import torch
    import fixed_order_fp_amd as bg
    print_case("gemm_reduce sliced", axis)
    M, N, K, LD = 45, 70, 24, 40
    Aw = synth.bf16_normal(901, (M, LD))
    Bw = synth.bf16_normal(902, (N, LD), sigma=0.05)
    big = synth.f32_to_bf16_bits(np.float32(1e30))
    Aw[:, K:] = big
    Bw[:, K:] = big
    A, B = np.ascontiguousarray(Aw[:, :K]), np.ascontiguousarray(Bw[:, :K])
    C32, (rs, rq) = oracle_ref(A, B, axis)
    d = bg.gemm_desc({"mfma": "F32_32X32X16_BF16"}, out_type="fp32")
    rd = bg.reduce_desc({"in_type": "fp32", "axis": axis, "op": "sum_and_sumsq"})
    dA, dB = to_dev_u16(Aw)[:, :K], to_dev_u16(Bw)[:, :K]
    dC = torch.empty((M, 72), dtype=torch.float32, device="cuda")[:, :N]
    n_out = N if axis == "col" else M
    s = torch.empty(n_out, dtype=torch.float32, device="cuda")
    q = torch.empty(n_out, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(bg.gemm_bf16_reduce_workspace_bytes(d, rd, M, N, K), 4) // 4, dtype=torch.float32,
                     device="cuda")
    bg.gemm_bf16_reduce(d, rd, dA, dB, dC, s, q, ws)
    dC2 = torch.empty((M, 72), dtype=torch.float32, device="cuda")[:, :N]
    bg.gemm_bf16(d, dA, dB, dC2, None)
    torch.cuda.synchronize()
    assert same(dC.cpu().numpy(), C32) and same(dC2.cpu().numpy(), C32)
    assert same(s.cpu().numpy(), rs) and same(q.cpu().numpy(), rq)
