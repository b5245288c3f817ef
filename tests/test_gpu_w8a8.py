"""GPU tests of the W8A8 power-of-two-scale GEMM through the C ABI.

The int32 accumulator must equal the oracle's exact integer sum and the bf16
output must match the oracle's fixed epilogue bit for bit, for every compiled
tile and both int8 instructions, at the full 1024 x 6144 x 2048 workload and
on ragged shapes whose K leaves a partial 128-byte tile."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import from_dev_u16, print_case, require_gpu

pytestmark = pytest.mark.gpu

# (instruction, bm, bn, waves_m, waves_n, load path, stages): path 2 is the
# pipelined kernel (two or three stages: 128-byte k tiles; four or more:
# 64-byte ones), path 1 the double-buffered one
TILES = [("I32_32X32X32_I8", 128, 192, 4, 2, 2, 2), ("I32_32X32X32_I8", 128, 192, 4, 2, 2, 3),
         ("I32_32X32X32_I8", 256, 256, 2, 4, 2, 2),
         ("I32_32X32X32_I8", 128, 128, 2, 2, 2, 2),
         ("I32_32X32X32_I8", 128, 128, 2, 2, 2, 4), ("I32_32X32X32_I8", 128, 128, 2, 2, 2, 5),
         ("I32_32X32X32_I8", 256, 256, 2, 4, 2, 4), ("I32_32X32X32_I8", 128, 192, 2, 2, 2, 4),
         ("I32_32X32X32_I8", 128, 192, 2, 2, 2, 5), ("I32_32X32X32_I8", 128, 192, 2, 2, 2, 6),
         ("I32_32X32X32_I8", 128, 192, 4, 2, 2, 5), ("I32_32X32X32_I8", 128, 64, 2, 2, 2, 8),
         ("I32_32X32X32_I8", 64, 64, 2, 2, 2, 8),
         ("I32_32X32X32_I8", 128, 128, 2, 2, 1, 0), ("I32_32X32X32_I8", 256, 128, 2, 2, 1, 0),
         ("I32_32X32X32_I8", 64, 64, 2, 2, 1, 0),
         ("I32_16X16X64_I8", 128, 128, 2, 2, 1, 0), ("I32_16X16X64_I8", 64, 64, 2, 2, 1, 0)]
TILE_IDS = [f"{t[0][4:13]}-{t[1]}x{t[2]}-w{t[3]}x{t[4]}-p{t[5]}-s{t[6]}" for t in TILES]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pad(n, q):
    return (n + q - 1) // q * q


def run_w8a8(a_q, w_q, a_scale, w_scale, instr="I32_32X32X32_I8", tile=None, want_acc=True):
    """Operands are copied into buffers whose leading dimensions are padded to
    the required multiples, so K need not be one.  Returns (Y bits, acc)."""
    import torch
    import fixed_order_fp_amd as bg
    M, K = a_q.shape
    N = w_q.shape[0]
    sched = {} if tile is None else dict(bm=tile[0], bn=tile[1], waves_m=tile[2], waves_n=tile[3],
                                         load_path=tile[4], stages=tile[5])
    d = bg.gemm_desc(dict(mfma=instr, a_type="int8", b_type="int8", acc_type="int32", out_type="bf16",
                          epilogue="W8A8_POW2", split_k=1, schedule=sched))
    kp = _pad(K, 16)
    dA = torch.zeros((M, kp), dtype=torch.int8, device="cuda")
    dW = torch.zeros((N, kp), dtype=torch.int8, device="cuda")
    dA[:, :K] = torch.from_numpy(np.ascontiguousarray(a_q)).cuda()
    dW[:, :K] = torch.from_numpy(np.ascontiguousarray(w_q)).cuda()
    # the padding columns hold a value that would show if the kernel read past K
    if kp > K:
        dA[:, K:] = 77
        dW[:, K:] = -91
    sa = torch.from_numpy(np.ascontiguousarray(a_scale, dtype=np.float32)).cuda()
    sw = torch.from_numpy(np.ascontiguousarray(w_scale, dtype=np.float32)).cuda()
    npad = _pad(N, 8)
    dY = torch.full((M, npad), 0x7FC1, dtype=torch.int16, device="cuda")
    dacc = torch.full((M, _pad(N, 4)), -7, dtype=torch.int32, device="cuda") if want_acc else None
    bg.gemm_w8a8_pow2(d, dA[:, :K], dW[:, :K], sa, sw, dY[:, :N],
                      None if dacc is None else dacc[:, :N])
    torch.cuda.synchronize()
    Y = from_dev_u16(dY)
    assert (Y[:, N:] == 0x7FC1).all(), "wrote past column N of Y"
    acc = None
    if dacc is not None:
        acc = dacc.cpu().numpy()
        assert (acc[:, N:] == -7).all(), "wrote past column N of acc"
        acc = acc[:, :N]
    return Y[:, :N], acc


def check(a_q, w_q, a_scale, w_scale, **kw):
    Y, acc = run_w8a8(a_q, w_q, a_scale, w_scale, **kw)
    Yo, acco = oracle.w8a8_pow2(a_q, w_q, a_scale, w_scale)
    if acc is not None:
        bad = np.argwhere(acc != acco)
        assert bad.size == 0, f"{len(bad)} int32 mismatches, first at {bad[0]}"
    bad = np.argwhere(Y != Yo)
    assert bad.size == 0, f"{len(bad)} bf16 mismatches, first at {bad[0]}: {Y[tuple(bad[0])]:#06x} vs {Yo[tuple(bad[0])]:#06x}"


def test_full_workload_default_schedule():
    a_q, w_q, a_s, w_s = synth.w8a8_input()
    print_case("w8a8 full", a_q.shape, w_q.shape)
    check(a_q, w_q, a_s, w_s)


@pytest.mark.parametrize("tile", TILES, ids=TILE_IDS)
def test_full_workload_every_tile(tile):
    a_q, w_q, a_s, w_s = synth.w8a8_input()
    print_case("w8a8 full tile", tile)
    check(a_q, w_q, a_s, w_s, instr=tile[0], tile=tile[1:], want_acc=False)


@pytest.mark.parametrize("tile", TILES, ids=TILE_IDS)
@pytest.mark.parametrize("M,N,K", [(200, 136, 2128), (1, 8, 16), (37, 300, 1), (130, 129, 333), (257, 64, 4100)])
def test_ragged(tile, M, N, K):
    instr = tile[0]
    a_q, _ = synth.quantize_per_token(synth.f32_normal(1100 + K, (M, K)))
    w_q = synth.int8_uniform(2100 + K, (N, K))
    w_s = synth.pow2_scales(3100 + K, N)
    _, a_s = synth.quantize_per_token(synth.f32_normal(1100 + K, (M, K)))
    print_case("w8a8 ragged", tile, M, N, K)
    check(a_q, w_q, a_s, w_s, instr=instr, tile=tile[1:])


def test_extreme_operands_max_k():
    """Every product is (-128)(-128) = 2^14 and K = 131071 (the largest K the
    entry point accepts): acc = 2^31 - 2^14, the top of the exact range."""
    M, N, K = 5, 9, 131071
    a_q = np.full((M, K), -128, dtype=np.int8)
    w_q = np.full((N, K), -128, dtype=np.int8)
    a_s = np.full(M, 1.0 / 127, dtype=np.float32)
    w_s = synth.pow2_scales(3200, N)
    print_case("w8a8 extreme", M, N, K)
    for tile in ((64, 64, 2, 2, 1, 0), (64, 64, 2, 2, 2, 8), (128, 128, 2, 2, 2, 4)):
        Y, acc = run_w8a8(a_q, w_q, a_s, w_s, tile=tile)
        assert (acc == K * 16384).all(), tile
        check(a_q, w_q, a_s, w_s, tile=tile)


def test_zero_rows_and_signed_extremes():
    """All-zero activation rows (scale 1), rows of +127 / -127 / -128, and
    alternating signs that cancel exactly."""
    M, N, K = 70, 96, 640
    rng = np.random.default_rng(4000)
    a_q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    a_q[0] = 0
    a_q[1] = 127
    a_q[2] = -127
    a_q[3] = -128
    a_q[4, 0::2], a_q[4, 1::2] = 100, -100
    w_q = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    w_q[5] = 1
    a_s = np.ldexp(rng.random(M).astype(np.float32) + 0.5, -7).astype(np.float32)
    a_s[0] = 1.0
    w_s = synth.pow2_scales(3300, N)
    for tile in TILES:
        print_case("w8a8 extremes", tile)
        check(a_q, w_q, a_s, w_s, instr=tile[0], tile=tile[1:])


def test_batch_invariance():
    """Row i of Y is the same bits whether the batch holds 1, 8, 64, 512 or
    1024 rows."""
    a_q, w_q, a_s, w_s = synth.w8a8_input()
    full, _ = run_w8a8(a_q, w_q, a_s, w_s, want_acc=False)
    for m in (1, 8, 64, 512):
        print_case("w8a8 batch", m)
        part, _ = run_w8a8(a_q[:m], w_q, a_s[:m], w_s, want_acc=False)
        assert np.array_equal(part, full[:m])


def test_free_order_epilogue_twin_gives_the_same_bits():
    """The bench's free-order twin (same main loop, the two scales combined
    before the multiply) returns the fixed epilogue's bits when the weight
    scales are powers of two ([W] section II: power-of-two commutation)."""
    import torch
    import fixed_order_fp_amd as bg
    a_q, w_q, a_s, w_s = synth.w8a8_input(M=200, N=320, K=512)
    print_case("w8a8 free twin 200x320x512")
    d = bg.gemm_desc(dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32",
                          out_type="bf16", epilogue="W8A8_POW2"))
    dA, dW = torch.from_numpy(a_q).cuda(), torch.from_numpy(w_q).cuda()
    sa, sw = torch.from_numpy(a_s).cuda(), torch.from_numpy(w_s).cuda()
    Y = torch.empty((200, 320), dtype=torch.int16, device="cuda")
    Yf = torch.full((200, 320), 7, dtype=torch.int16, device="cuda")
    bg.gemm_w8a8_pow2(d, dA, dW, sa, sw, Y)
    bg.bench_gemm_w8a8_free(dA, dW, sa, sw, Yf)
    torch.cuda.synchronize()
    assert torch.equal(Y, Yf)
