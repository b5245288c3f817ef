"""The measured instruction model against the hardware, on fresh draws.

The MFMA profile was chosen by the black-box probe ('Taming Bitwise
Behavior', section 4, applied to one instruction).  Here one million random
single instructions per bf16 instruction, drawn with seeds the fit never saw
(ordinary, exponent-spread, cancelling, far accumulators), must match the
oracle evaluating that profile bit for bit; the int8 instructions must return
the exact int32 sum."""
import numpy as np
import pytest

import synth
from gpu_util import measured_model, print_case, require_gpu

pytestmark = pytest.mark.gpu

SHAPES = {"F32_32X32X16_BF16": (32, 16), "F32_16X16X32_BF16": (16, 32)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run_probe(instr, A, B, Cm):
    import torch
    import fixed_order_fp_amd as bg
    dA = torch.from_numpy(A.view(np.int16).copy()).cuda()
    dB = torch.from_numpy(B.view(np.int16).copy()).cuda()
    dC = torch.from_numpy(np.ascontiguousarray(Cm)).cuda()
    dD = torch.empty_like(dC)
    bg.probe_mfma(instr, A.shape[0], dA, dB, dC, dD)
    torch.cuda.synchronize()
    return dD.cpu().numpy()


def _draws(instr, seed, n_out):
    R, K = SHAPES[instr]
    W = n_out // (R * R) // 4
    rng = np.random.default_rng(seed)
    parts = []
    # ordinary
    parts.append((synth.bf16_normal(seed + 1, (W, R, K)), synth.bf16_normal(seed + 2, (W, R, K)),
                  synth.f32_normal(seed + 3, (W, R, R), 0.0, 3.0)))
    # exponent spread
    parts.append((synth.bf16_spread(seed + 4, (W, R, K), -30, 30), synth.bf16_spread(seed + 5, (W, R, K), -30, 30),
                  synth.f32_spread(seed + 6, (W, R, R), -60, 60)))
    # cancellation
    A = synth.bf16_spread(seed + 7, (W, R, K), -12, 12)
    A[:, :, K // 2:] = A[:, :, :K // 2] ^ 0x8000
    A[:, :, :2] = synth.bf16_spread(seed + 8, (W, R, 2), -40, -10)
    A = np.take_along_axis(A, rng.permuted(np.tile(np.arange(K), (W, R, 1)), axis=2), axis=2)
    parts.append((A, synth.bf16_spread(seed + 9, (W, R, K), -2, 2), synth.f32_spread(seed + 10, (W, R, R), -30, 10)))
    # accumulator far from the products
    ex = rng.integers(-40, 45, size=(W, R, R))
    Cm = (np.ldexp(1.0, ex) * (1 + rng.random((W, R, R)))).astype(np.float32)
    parts.append((synth.bf16_normal(seed + 11, (W, R, K)), synth.bf16_normal(seed + 12, (W, R, K)), Cm))
    return parts


@pytest.mark.parametrize("instr", list(SHAPES))
def test_random_instructions_match_the_profile(instr):
    import oracle
    model = measured_model(instr)
    R, K = SHAPES[instr]
    total = 0
    for A, B, Cm in _draws(instr, 7000 + K, 1 << 20):
        print_case("probe_random", instr, A.shape)
        D = _run_probe(instr, A, B, Cm)
        acc = Cm.reshape(-1)
        a = np.repeat(A[:, :, None, :], R, axis=2).reshape(-1, K)
        b = np.repeat(B[:, None, :, :], R, axis=1).reshape(-1, K)
        ref = oracle.mfma_bf16_batch(model, acc, a, b)
        bad = np.sum(ref.view(np.uint32) != D.reshape(-1).view(np.uint32))
        assert bad == 0, f"{bad} of {acc.size} outputs differ from the profile"
        total += acc.size
    assert total >= 1_000_000


@pytest.mark.parametrize("instr,R,K", [("I32_32X32X32_I8", 32, 32), ("I32_16X16X64_I8", 16, 64)])
def test_int8_instructions_are_exact(instr, R, K):
    import torch
    import fixed_order_fp_amd as bg
    print_case("probe_int8", instr)
    rng = np.random.default_rng(11)
    W = 256
    A = rng.integers(-128, 128, size=(W, R, K)).astype(np.int8)
    B = rng.integers(-128, 128, size=(W, R, K)).astype(np.int8)
    Cm = rng.integers(-(1 << 30), 1 << 30, size=(W, R, R)).astype(np.int32)
    dA, dB, dC = (torch.from_numpy(x).cuda() for x in (A, B, Cm))
    dD = torch.empty_like(dC)
    bg.probe_mfma(instr, W, dA, dB, dC, dD)
    torch.cuda.synchronize()
    exact = Cm.astype(np.int64) + np.einsum("wmk,wnk->wmn", A.astype(np.int64), B.astype(np.int64))
    assert np.array_equal(dD.cpu().numpy().astype(np.int64), exact)


@pytest.mark.parametrize("instr", list(SHAPES))
def test_zero_products_leave_tiny_accumulators_alone(instr):
    """The short last turn of a walk, and the extra k-steps of the 64-deep
    register and direct-load kernels' last turn, issue instructions whose
    every product is +0 or -0.  Fresh draws of such instructions against
    accumulators at the bottom of the fp32 range -- subnormals of every
    size, near-underflow normals, signed zeros -- must match the profile
    (which returns the accumulator unchanged) bit for bit."""
    import oracle
    model = measured_model(instr)
    R, K = SHAPES[instr]
    rng = np.random.default_rng(9100 + K)
    W = 512
    # products of +-0 with anything finite, and of anything with +-0
    A = np.where(rng.random((W, R, K)) < 0.5, 0x8000, 0x0000).astype(np.uint16)
    B = synth.bf16_spread(9101 + K, (W, R, K), -60, 60)
    half = W // 2
    A[half:], B[half:] = B[half:].copy(), np.where(rng.random((W - half, R, K)) < 0.5, 0x8000, 0x0000).astype(np.uint16)
    sub = (rng.integers(1, 1 << 23, size=(W, R, R)).astype(np.uint32)
           | (rng.integers(0, 2, size=(W, R, R)).astype(np.uint32) << 31))
    near = synth.f32_spread(9102 + K, (W, R, R), -126, -110)
    zeros = np.where(rng.random((W, R, R)) < 0.5, -0.0, 0.0).astype(np.float32)
    pick = rng.integers(0, 3, size=(W, R, R))
    Cm = np.where(pick == 0, sub.view(np.float32), np.where(pick == 1, near, zeros)).astype(np.float32)
    print_case("probe_zero_products", instr, A.shape)
    D = _run_probe(instr, A, B, Cm)
    acc = Cm.reshape(-1)
    a = np.repeat(A[:, :, None, :], R, axis=2).reshape(-1, K)
    b = np.repeat(B[:, None, :, :], R, axis=1).reshape(-1, K)
    ref = oracle.mfma_bf16_batch(model, acc, a, b)
    assert np.array_equal(ref.view(np.uint32), D.reshape(-1).view(np.uint32))
    # and the profile's reading: the accumulator passes through unchanged,
    # except that -0 plus a +0 product is +0 (IEEE round-to-nearest)
    moved = D.reshape(-1).view(np.uint32) != acc.view(np.uint32)
    assert np.all(acc[moved] == 0)

