"""GPU tests of the Ozaki-scheme GEMM (bg_gemm_ozaki) through the C ABI, bit
for bit against the oracle's Ozaki GEMM: fp32 and bf16 operands and outputs,
ragged K (a zero-padded k tail), wide exponent spreads (slices that drop
bits, dropped identically on both sides), zero rows, and the headline shape
on sampled rows and columns (the slicing is per row, so a sub-matrix of the
operands gives the same outputs).  Permuting k must not move a bit."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import from_dev_u16, print_case, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run(A, B, in_type, out_type):
    import torch
    import fixed_order_fp_amd as bg
    M, K = A.shape
    N = B.shape[0]
    if in_type == "bf16":
        dA = torch.from_numpy(np.ascontiguousarray(A).view(np.int16)).cuda()
        dB = torch.from_numpy(np.ascontiguousarray(B).view(np.int16)).cuda()
    else:
        dA, dB = torch.from_numpy(np.ascontiguousarray(A)).cuda(), torch.from_numpy(np.ascontiguousarray(B)).cuda()
    ldc = N + 3
    dC = torch.full((M, ldc), -7, dtype=torch.float32 if out_type == "fp32" else torch.int16, device="cuda")
    ws = torch.empty(bg.gemm_ozaki_workspace_bytes(M, N, K) // 4 + 4, dtype=torch.float32, device="cuda")
    bg.gemm_ozaki(dA, dB, dC[:, :N], in_type, out_type, ws)
    torch.cuda.synchronize()
    C = dC.cpu().numpy()
    assert (C[:, N:] == -7).all(), "wrote past column N"
    C = C[:, :N]
    return np.ascontiguousarray(C) if out_type == "fp32" else np.ascontiguousarray(C).view(np.uint16)


def check(A, B, in_type, out_type):
    C = run(A, B, in_type, out_type)
    Co = oracle.ozaki_gemm(A, B, in_type=in_type, out_type=out_type)
    bad = np.argwhere(C.view(np.uint16 if out_type == "bf16" else np.uint32) !=
                      Co.view(np.uint16 if out_type == "bf16" else np.uint32))
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0]}"
    return C


@pytest.mark.parametrize("in_type,out_type", [("fp32", "fp32"), ("fp32", "bf16"), ("bf16", "fp32"),
                                              ("bf16", "bf16")])
@pytest.mark.parametrize("M,N,K", [(64, 96, 128), (33, 70, 17), (1, 40, 1000), (130, 257, 100), (5, 3, 1)])
def test_against_oracle(in_type, out_type, M, N, K):
    print_case("ozaki", in_type, out_type, M, N, K)
    if in_type == "bf16":
        A, B = synth.bf16_normal(10 + M, (M, K)), synth.bf16_normal(20 + N, (N, K), sigma=0.02)
    else:
        A, B = synth.f32_normal(10 + M, (M, K)), synth.f32_normal(20 + N, (N, K), sigma=0.02)
    check(A, B, in_type, out_type)


@pytest.mark.parametrize("M,N,K,out_type", [(500, 1000, 300, "fp32"), (260, 3000, 200, "bf16")])
def test_mid_size_tiles(M, N, K, out_type):
    """Stacked products large enough for the 128-row int8 tiles (the
    recombination runs in every tile's epilogue), ragged M and N."""
    print_case("ozaki mid", M, N, K, out_type)
    A, B = synth.f32_spread(60 + M, (M, K), -12, 12), synth.f32_spread(61 + N, (N, K), -12, 12)
    check(A, B, "fp32", out_type)


def test_wide_spread_and_zero_rows():
    """Exponents over +-30 (the slices keep 28 bits below each row's largest),
    zero rows in both operands."""
    print_case("ozaki spread")
    A = synth.f32_spread(31, (40, 300), -30, 30)
    B = synth.f32_spread(32, (50, 300), -30, 30)
    A[3] = 0.0
    B[7] = 0.0
    check(A, B, "fp32", "fp32")


def test_deepest_k():
    """K = 133,133, padded to 133,136: the deepest padded k (a multiple of
    16) whose slice products still sum exactly in int32 (K 127^2 < 2^31)."""
    print_case("ozaki deepest k")
    A = synth.f32_spread(51, (3, 133133), -8, 8)
    B = synth.f32_spread(52, (5, 133133), -8, 8)
    check(A, B, "fp32", "fp32")


def test_k_order_does_not_move_a_bit():
    print_case("ozaki k order")
    A = synth.f32_spread(41, (64, 512), -10, 10)
    B = synth.f32_spread(42, (80, 512), -10, 10)
    C = run(A, B, "fp32", "fp32")
    p = np.random.default_rng(0).permutation(512)
    Cp = run(np.ascontiguousarray(A[:, p]), np.ascontiguousarray(B[:, p]), "fp32", "fp32")
    assert np.array_equal(C.view(np.uint32), Cp.view(np.uint32))


def test_headline_shape_sampled():
    """M=4000, N=9728, K=2560 bf16 (the batch-sweep operands) to bf16, checked
    on 32 rows x 128 columns (the first and last of each included) through
    the oracle on those rows and columns."""
    print_case("ozaki headline")
    X, W = synth.gemm_batch_sweep(M=4000)
    C = run(X, W, "bf16", "bf16")
    rng = np.random.default_rng(4)
    mi = np.sort(np.concatenate([rng.choice(4000, 30, replace=False), [0, 3999]]))
    ni = np.sort(np.concatenate([rng.choice(9728, 126, replace=False), [0, 9727]]))
    Co = oracle.ozaki_gemm(X[mi], W[ni], in_type="bf16", out_type="bf16")
    assert np.array_equal(C[np.ix_(mi, ni)], Co)


def test_argument_errors():
    import torch
    import fixed_order_fp_amd as bg
    A = torch.zeros((8, 16), dtype=torch.float32, device="cuda")
    Cc = torch.zeros((8, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(bg.BgError):   # no workspace
        bg.gemm_ozaki(A, A, Cc, "fp32", "fp32", None)
    # K past the int32 bound: refused before anything is read
    assert bg.lib().bg_gemm_ozaki(8, 8, 200000, 0, A.data_ptr(), 200000, A.data_ptr(), 200000, 0, Cc.data_ptr(), 8,
                                  None, 0, None) != 0
