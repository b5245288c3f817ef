"""GPU tests of the int8 quantisation on either side of W8A8 through the C ABI:
per-token activation quantisation and requantisation of int8 weights to
power-of-two scales, bit for bit against the oracle (codes and scales), on the
vector and the scalar paths, ragged rows, padded leading dimensions, zero
rows, exact halves, extreme and non-finite values; then the whole chain
(fp32 activations and weights with free scales -> int8 -> W8A8) against the
oracle's chain."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import from_dev_u16, print_case, require_gpu

pytestmark = pytest.mark.gpu

SENT = 0x5A


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_quantize(X, pad=0, offset=0):
    """X fp32 [M][K] on the device with `offset` leading floats per row (so the
    row start can be unaligned) and `pad` extra columns; Q with a sentinel in
    its padding.  Returns (Q, scale)."""
    import torch
    import fixed_order_fp_amd as bg
    M, K = X.shape
    dX = torch.zeros((M, offset + K + pad), dtype=torch.float32, device="cuda")
    dX[:, offset:offset + K] = torch.from_numpy(np.ascontiguousarray(X, dtype=np.float32)).cuda()
    if pad:
        dX[:, offset + K:] = 1e30  # would show in the scale if read
    dQ = torch.full((M, K + pad + 3), SENT, dtype=torch.int8, device="cuda")
    ds = torch.full((M + 1,), -5.0, dtype=torch.float32, device="cuda")
    bg.quantize_act_int8(dX[:, offset:offset + K], dQ[:, :K], ds[:M])
    torch.cuda.synchronize()
    Q = dQ.cpu().numpy()
    assert (Q[:, K:] == SENT).all(), "wrote past column K of Q"
    s = ds.cpu().numpy()
    assert s[M] == -5.0
    return Q[:, :K], s[:M]


def check_quantize(X, **kw):
    Q, s = run_quantize(X, **kw)
    Qo, so = oracle.quantize_rows_int8(X)
    assert np.array_equal(s.view(np.uint32), so.view(np.uint32)), "scale mismatch"
    bad = np.argwhere(Q != Qo)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0]}"


def test_workload_1024x2048():
    print_case("quantize", 1024, 2048)
    x = synth.f32_normal(1005, (1024, 2048))
    check_quantize(x)


@pytest.mark.parametrize("M,K,pad,offset", [(7, 1, 0, 0), (5, 3, 1, 0), (33, 2049, 0, 0), (9, 4097, 3, 1),
                                            (17, 256, 0, 1), (3, 1000, 24, 0), (2, 0, 0, 0), (1, 8192 + 4, 0, 0),
                                            (2, 8192, 0, 0), (7, 4096, 0, 0), (6, 4092, 4, 0), (5, 4, 0, 0)])
def test_ragged_and_unaligned(M, K, pad, offset):
    print_case("quantize ragged", M, K, pad, offset)
    x = synth.f32_spread(300 + K, (M, K), -20, 20) if K else np.zeros((M, 0), np.float32)
    check_quantize(x, pad=pad, offset=offset)


def test_zero_rows_halves_and_extremes():
    print_case("quantize special rows")
    K = 512
    rows = [np.zeros(K, np.float32)]
    k = np.arange(K - 1) % 253 - 126
    rows.append(np.concatenate([((k + 0.5) / 8.0), [127 / 8.0]]).astype(np.float32))   # exact halves
    rows.append(np.full(K, 1e-40, np.float32))                                         # subnormal
    rows.append(np.linspace(-3e38, 3e38, K).astype(np.float32))                        # near the top
    rows.append((np.arange(K) % 3 - 1).astype(np.float32) * np.float32(-0.0))          # signed zeros
    r = np.random.default_rng(9).standard_normal(K).astype(np.float32)
    r[17] = np.inf
    rows.append(r)
    r = np.random.default_rng(10).standard_normal(K).astype(np.float32)
    r[5] = np.nan
    rows.append(r)
    check_quantize(np.stack(rows))


def run_requant(W, s, mode, pad=0, offset=0):
    import torch
    import fixed_order_fp_amd as bg
    N, K = W.shape
    dW = torch.zeros((N, offset + K + pad), dtype=torch.int8, device="cuda")
    dW[:, offset:offset + K] = torch.from_numpy(np.ascontiguousarray(W, dtype=np.int8)).cuda()
    dO = torch.full((N, K + pad + 5), SENT, dtype=torch.int8, device="cuda")
    ds = torch.from_numpy(np.ascontiguousarray(s, dtype=np.float32)).cuda()
    do = torch.full((N + 1,), -5.0, dtype=torch.float32, device="cuda")
    bg.requantize_weights_pow2(dW[:, offset:offset + K], ds, dO[:, :K], do[:N], mode)
    torch.cuda.synchronize()
    O = dO.cpu().numpy()
    assert (O[:, K:] == SENT).all(), "wrote past column K"
    so = do.cpu().numpy()
    assert so[N] == -5.0
    return O[:, :K], so[:N]


def check_requant(W, s, mode, **kw):
    O, so = run_requant(W, s, mode, **kw)
    Oo, soo = oracle.requantize_pow2(W, s, mode)
    assert np.array_equal(so.view(np.uint32), soo.view(np.uint32)), "scale mismatch"
    bad = np.argwhere(O != Oo)
    assert bad.size == 0, f"{len(bad)} weight mismatches, first at {bad[0]}"


@pytest.mark.parametrize("mode", ["nearest", "ceil"])
def test_requantize_6144x2048(mode):
    print_case("requantize", mode, 6144, 2048)
    W = synth.int8_uniform(2005, (6144, 2048))
    s = np.exp(np.random.default_rng(11).uniform(-9, -3, 6144)).astype(np.float32)
    check_requant(W, s, mode)


@pytest.mark.parametrize("mode", ["nearest", "ceil"])
@pytest.mark.parametrize("N,K,pad,offset", [(5, 1, 0, 0), (9, 17, 3, 1), (33, 100, 0, 0), (4, 4096 + 16, 16, 0),
                                            (3, 0, 0, 0), (7, 48, 16, 0), (1001, 16, 0, 0)])
def test_requantize_ragged(mode, N, K, pad, offset):
    print_case("requantize ragged", mode, N, K, pad, offset)
    W = synth.int8_uniform(400 + K, (N, K))
    s = np.exp(np.random.default_rng(12 + K).uniform(-20, 5, N)).astype(np.float32)
    check_requant(W, s, mode, pad=pad, offset=offset)


@pytest.mark.parametrize("mode", ["nearest", "ceil"])
def test_requantize_special_scales(mode):
    """Powers of two, the floats around sqrt 2, a subnormal, the largest
    finite scale (rounds up to infinity), and unusable scales."""
    print_case("requantize special", mode)
    s = np.array([0.5, 2.0 ** -20, 1.41421353816986083984375, 1.41421365737915039062500, 1e-40,
                  3.4e38, 0.0, -1.0, np.inf, np.nan, 0.7, 0.75], dtype=np.float32)
    W = synth.int8_uniform(77, (len(s), 64))
    check_requant(W, s, mode)


def test_chain_into_w8a8():
    """fp32 activations and int8 weights with free scales -> per-token
    quantisation and power-of-two requantisation on the GPU -> W8A8 on the
    GPU, against the same chain in the oracle."""
    import torch
    import fixed_order_fp_amd as bg
    print_case("chain", 256, 512, 1024)
    M, N, K = 256, 512, 1024
    x = synth.f32_normal(31, (M, K))
    W = synth.int8_uniform(32, (N, K))
    s = np.exp(np.random.default_rng(33).uniform(-8, -4, N)).astype(np.float32)
    dX = torch.from_numpy(x).cuda()
    dQ = torch.empty((M, K), dtype=torch.int8, device="cuda")
    da = torch.empty(M, dtype=torch.float32, device="cuda")
    dW = torch.from_numpy(W).cuda()
    dW2 = torch.empty_like(dW)
    ds = torch.from_numpy(s).cuda()
    ds2 = torch.empty_like(ds)
    dY = torch.empty((M, N), dtype=torch.int16, device="cuda")
    d = bg.gemm_desc(dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32",
                          out_type="bf16", epilogue="W8A8_POW2"))
    bg.quantize_act_int8(dX, dQ, da)
    bg.requantize_weights_pow2(dW, ds, dW2, ds2, "nearest")
    bg.gemm_w8a8_pow2(d, dQ, dW2, da, ds2, dY)
    torch.cuda.synchronize()
    Qo, ao = oracle.quantize_rows_int8(x)
    W2o, s2o = oracle.requantize_pow2(W, s, "nearest")
    Yo, _ = oracle.w8a8_pow2(Qo, W2o, ao, s2o)
    assert np.array_equal(from_dev_u16(dY), Yo)


def test_argument_errors():
    import torch
    import fixed_order_fp_amd as bg
    X = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    Q = torch.zeros((4, 8), dtype=torch.int8, device="cuda")
    a = torch.zeros(4, dtype=torch.float32, device="cuda")
    lib = bg.lib()
    assert lib.bg_quantize_act_int8(-1, 8, X.data_ptr(), 8, Q.data_ptr(), 8, a.data_ptr(), None) != 0
    assert lib.bg_quantize_act_int8(4, 8, X.data_ptr(), 4, Q.data_ptr(), 8, a.data_ptr(), None) != 0
    assert lib.bg_quantize_act_int8(4, 8, None, 8, Q.data_ptr(), 8, a.data_ptr(), None) != 0
    assert lib.bg_quantize_act_int8(0, 8, None, 8, None, 8, None, None) == 0
    W = torch.zeros((4, 16), dtype=torch.int8, device="cuda")
    s = torch.ones(4, dtype=torch.float32, device="cuda")
    assert lib.bg_requantize_weights_pow2(4, 16, W.data_ptr(), 16, s.data_ptr(), 2, W.data_ptr() + 64 * 4, 16,
                                          s.data_ptr(), None) != 0                       # unknown mode
    assert lib.bg_requantize_weights_pow2(4, 16, W.data_ptr(), 16, s.data_ptr(), 0, W.data_ptr() + 8, 16,
                                          s.data_ptr(), None) != 0                       # overlap
