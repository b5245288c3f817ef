"""GPU tests of the fixed-order row and column reductions through the C ABI:
0 ULP against the oracle (leaves of 32 folded in index order, a balanced
neighbours-first tree over the leaves), at the workloads' full sizes and on
ragged shapes, plus invariance checks.  The free-order twins are checked
against the summation error bound only."""
import math

import numpy as np
import pytest

import synth
from gpu_util import print_case, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_reduce(X, axis, in_type, fused=True, op="sum_and_sumsq", cols=None, schedule=None):
    """X: numpy fp32 or bf16-bit array [rows][ld]; reduces the first `cols`
    columns.  Returns (sum, sumsq) numpy arrays."""
    import torch
    import fixed_order_fp_amd as bg
    rows, ld = X.shape
    cols = ld if cols is None else cols
    dX = torch.from_numpy(X.view(np.int16) if in_type == "bf16" else X).cuda()[:, :cols]
    n_out = rows if axis == "row" else cols
    d = bg.reduce_desc({"in_type": in_type, "axis": axis, "sq_fma": "fused" if fused else "unfused",
                        "op": op, "schedule": schedule or {}})
    s = torch.full((n_out,), float("nan"), dtype=torch.float32, device="cuda")
    q = torch.full((n_out,), float("nan"), dtype=torch.float32, device="cuda")
    nws = bg.reduce_workspace_bytes(d, rows, cols)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    bg.reduce_tree(d, dX, s, q, ws)
    torch.cuda.synchronize()
    return s.cpu().numpy(), q.cpu().numpy()


def oracle_reduce(X, axis, in_type, fused=True, cols=None):
    import oracle
    cols = X.shape[1] if cols is None else cols
    return oracle.reduce(np.ascontiguousarray(X[:, :cols]), axis, leaf_len=32, sq_fused=fused, in_type=in_type)


def same(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_row_sum_and_sumsq_full_workload():
    """16384 x 8192 fp32 ~ N(0,1): row sum and sum of squares in one pass,
    every output bit-identical to the oracle."""
    print_case("row_full")
    X = synth.reduce_rows_input()
    s, q = run_reduce(X, "row", "fp32")
    rs, rq = oracle_reduce(X, "row", "fp32")
    assert same(s, rs) and same(q, rq)


def test_col_sum_full_workload():
    """8192 x 4096 bf16 ~ N(0, 0.1): column sums (and squares), bit-identical
    to the oracle, for several workgroup shapes (speed knobs only)."""
    Y = synth.reduce_cols_input()
    rs, rq = oracle_reduce(Y, "col", "bf16")
    for sched in ({}, {"leaves_per_wg": 4}, {"leaves_per_wg": 16}, {"leaves_per_wg": 32},
                  {"leaves_per_wg": 8, "cols_per_wg": 512}, {"leaves_per_wg": 16, "cols_per_wg": 512}):
        print_case("col_full", sched)
        s, q = run_reduce(Y, "col", "bf16", schedule=sched)
        assert same(s, rs) and same(q, rq), sched


@pytest.mark.parametrize("in_type", ["fp32", "bf16"])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("rows,ld,cols", [(37, 8192, 8192), (5, 104, 100), (9, 72, 70), (3, 32, 32),
                                          (4, 20000, 20000), (2, 16384 + 8, 16390), (6, 8, 1)])
def test_row_ragged(in_type, fused, rows, ld, cols):
    """Short last leaves, odd leaf counts, several leaf blocks per row (a
    workspace and the second-level tree), a single leaf, a single element."""
    print_case("row_ragged", in_type, fused, rows, ld, cols)
    if in_type == "fp32":
        X = synth.f32_spread(77 + cols, (rows, ld), -12, 12)
    else:
        X = synth.bf16_spread(77 + cols, (rows, ld), -12, 12)
    s, q = run_reduce(X, "row", in_type, fused, cols=cols)
    rs, rq = oracle_reduce(X, "row", in_type, fused, cols=cols)
    assert same(s, rs) and same(q, rq)


@pytest.mark.parametrize("in_type", ["fp32", "bf16"])
@pytest.mark.parametrize("cols", [64 * 8192, 64 * 8192 - 5])
def test_row_longest(in_type, cols):
    """The longest row built: 64 blocks of 256 leaves (a full second-level
    tree of 64 block roots), and the same with a short last leaf."""
    print_case("row_longest", in_type, cols)
    ld = (cols + 7) // 8 * 8
    X = synth.f32_spread(301, (2, ld), -12, 12) if in_type == "fp32" else synth.bf16_spread(301, (2, ld), -12, 12)
    s, q = run_reduce(X, "row", in_type, cols=cols)
    rs, rq = oracle_reduce(X, "row", in_type, cols=cols)
    assert same(s, rs) and same(q, rq)


@pytest.mark.parametrize("in_type", ["fp32", "bf16"])
@pytest.mark.parametrize("rows", [65536, 65536 - 7])
def test_col_deepest(in_type, rows):
    """The longest column built on the default path: 2048 leaves, 32 leaves
    per workgroup (the default raised until 64 block roots remain), and the
    same with a short last leaf."""
    print_case("col_deepest", in_type, rows)
    X = synth.f32_spread(302, (rows, 40), -12, 12) if in_type == "fp32" else synth.bf16_spread(302, (rows, 40), -12, 12)
    s, q = run_reduce(X, "col", in_type, cols=36)
    rs, rq = oracle_reduce(X, "col", in_type, cols=36)
    assert same(s, rs) and same(q, rq)


@pytest.mark.parametrize("in_type", ["fp32", "bf16"])
@pytest.mark.parametrize("rows,ld,cols,lpw", [(1000, 304, 300, 8), (8192, 256, 256, 32), (33, 8, 5, 4),
                                              (4096 + 32 * 3 + 7, 520, 513, 16), (32, 256, 256, 8)])
def test_col_ragged(in_type, rows, ld, cols, lpw):
    print_case("col_ragged", in_type, rows, cols, lpw)
    if in_type == "fp32":
        X = synth.f32_spread(99 + rows, (rows, ld), -12, 12)
    else:
        X = synth.bf16_spread(99 + rows, (rows, ld), -12, 12)
    s, q = run_reduce(X, "col", in_type, True, cols=cols, schedule={"leaves_per_wg": lpw})
    rs, rq = oracle_reduce(X, "col", in_type, True, cols=cols)
    assert same(s, rs) and same(q, rq)


@pytest.mark.parametrize("in_type", ["fp32", "bf16"])
@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("rows,ld,cols", [(1000, 304, 300), (8192, 256, 256), (33, 8, 5), (4096 + 32 * 3 + 7, 520, 513),
                                          (32, 256, 256), (8192, 4104, 4100), (8191, 40, 33), (1, 16, 3),
                                          (8193, 64, 64)])
def test_col_ragged_default_and_one_pass(in_type, fused, rows, ld, cols):
    """The default column path (two kernels) and the one-pass path (a
    workgroup per column strip over every row, rows <= 8192): short last
    leaves, odd leaf counts, ragged strips, a single row."""
    print_case("col_ragged_default", in_type, fused, rows, cols)
    if in_type == "fp32":
        X = synth.f32_spread(199 + rows, (rows, ld), -12, 12)
    else:
        X = synth.bf16_spread(199 + rows, (rows, ld), -12, 12)
    rs, rq = oracle_reduce(X, "col", in_type, fused, cols=cols)
    s, q = run_reduce(X, "col", in_type, fused, cols=cols)
    assert same(s, rs) and same(q, rq)
    if rows <= 8192:
        s, q = run_reduce(X, "col", in_type, fused, cols=cols, schedule={"leaves_per_wg": 256})
        assert same(s, rs) and same(q, rq)


def test_ops_write_only_what_they_ask_for():
    X = synth.f32_normal(5, (16, 8192))
    s, q = run_reduce(X, "row", "fp32", op="sum")
    assert not np.isnan(s).any() and np.isnan(q).all()
    s, q = run_reduce(X, "row", "fp32", op="sumsq")
    assert np.isnan(s).all() and not np.isnan(q).any()


def test_row_result_does_not_depend_on_other_rows():
    """A row's bits are the same whatever else is in the batch."""
    X = synth.f32_spread(3, (64, 8192), -10, 10)
    s_all, q_all = run_reduce(X, "row", "fp32")
    s_one, q_one = run_reduce(np.ascontiguousarray(X[17:18]), "row", "fp32")
    assert same(s_all[17:18], s_one) and same(q_all[17:18], q_one)


@pytest.mark.parametrize("axis", ["row", "col"])
def test_free_order_twins_obey_the_error_bound(axis):
    """No bitwise contract: |y - exact| <= gamma_{n-1} sum |x|."""
    import torch
    import fixed_order_fp_amd as bg
    X = synth.f32_normal(11, (512, 4096)) if axis == "row" else synth.f32_normal(12, (4096, 512))
    dX = torch.from_numpy(X).cuda()
    n_out = X.shape[0] if axis == "row" else X.shape[1]
    s = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    q = torch.zeros(n_out, dtype=torch.float32, device="cuda")
    bg.bench_reduce_free(axis, "fp32", dX, s, q)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    n = X.shape[1] if axis == "row" else X.shape[0]
    u = 2.0 ** -24
    g = (n - 1) * u / (1 - (n - 1) * u)
    V = X if axis == "row" else X.T
    for i in range(0, n_out, 7):
        exact = math.fsum(V[i].astype(np.float64))
        assert abs(float(s[i]) - exact) <= g * float(np.abs(V[i].astype(np.float64)).sum())
