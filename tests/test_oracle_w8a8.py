"""Pins for the oracle's W8A8 path with power-of-two weight scales
('Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
Quantization Scales', section II: Y = (A W^T) s_a s_w with exact INT32
accumulation, and the power-of-two commutation)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from exact import f32_value, round_bf16_bits, round_f32


@pytest.fixture(scope="module")
def small():
    # the workload's recipe at a size the oracle finishes in a moment
    x = synth.f32_normal(1005, (96, 2048))
    a_q, a_s = synth.quantize_per_token(x)
    w_q = synth.int8_uniform(2005, (160, 2048))
    w_s = synth.pow2_scales(3005, 160)
    return a_q, w_q, a_s, w_s


def test_int32_accumulator_is_the_exact_integer(small):
    a_q, w_q, a_s, w_s = small
    _, acc = oracle.w8a8_pow2(a_q, w_q, a_s, w_s)
    ref = a_q.astype(np.int64) @ w_q.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), ref)


def test_int32_bound_holds_at_full_depth():
    """|acc| <= K * 127 * 127 = 33,032,192 < 2^31 at K = 2048, reached by
    all-(+-127) operands."""
    a = np.full((2, 2048), 127, dtype=np.int8)
    w = np.full((3, 2048), -127, dtype=np.int8)
    _, acc = oracle.w8a8_pow2(a, w, np.ones(2, np.float32), np.ones(3, np.float32))
    assert np.all(acc == -2048 * 127 * 127)


def test_epilogue_is_the_stated_double_rounding(small):
    """y = bf16_RNE( fp32_RNE( fp32_RNE(acc) * w_scale ) * a_scale ), checked
    with exact rationals and an independent correct rounding."""
    a_q, w_q, a_s, w_s = small
    y, acc = oracle.w8a8_pow2(a_q, w_q, a_s, w_s)
    rng = np.random.default_rng(2)
    for m, n in zip(rng.integers(0, 96, 400), rng.integers(0, 160, 400)):
        f = round_f32(Fraction(int(acc[m, n])))
        t = round_f32(f32_value(f) * f32_value(w_s[n]))
        u = round_f32(f32_value(t) * f32_value(a_s[m]))
        assert int(y[m, n]) == round_bf16_bits(f32_value(u))


def test_large_accumulators_round_to_nearest_even():
    """Above 2^24 the int->fp32 conversion rounds (ties to even)."""
    a = np.zeros((1, 2048), dtype=np.int8)
    w = np.zeros((1, 2048), dtype=np.int8)
    a[0, :1041] = 127
    w[0, :1041] = 127
    a[0, 1041] = 1
    w[0, 1041] = 1  # acc = 1041*16129 + 1 = 16,790,290 (even + 1 -> rounds)
    y, acc = oracle.w8a8_pow2(a, w, np.ones(1, np.float32), np.ones(1, np.float32))
    assert acc[0, 0] == 1041 * 16129 + 1
    assert synth.bf16_bits_to_f32(y)[0, 0] == synth.bf16_bits_to_f32(
        round_bf16_bits(f32_value(round_f32(Fraction(int(acc[0, 0]))))))


def test_power_of_two_commutation(small):
    """With power-of-two weight scales the two legal multiplication orders are
    bit-identical before the bf16 cast (finite normal values)."""
    a_q, w_q, a_s, w_s = small
    _, acc = oracle.w8a8_pow2(a_q, w_q, a_s, w_s)
    f = acc.astype(np.float32)
    ws_first = (f * w_s[None, :]) * a_s[:, None]
    as_first = (f * a_s[:, None]) * w_s[None, :]
    assert np.array_equal(ws_first.view(np.uint32), as_first.view(np.uint32))


def _epilogue_variants(acc, a_s, w_s):
    """The stated epilogue and planted faults (on the CPU only)."""
    f = acc.astype(np.float32)
    ref = oracle.bf16_rne((f * w_s[None, :]) * a_s[:, None])
    faults = {}
    # scale precision: the activation scale held in bf16
    a_bf = synth.bf16_bits_to_f32(oracle.bf16_rne(a_s))
    faults["scale_precision"] = oracle.bf16_rne((f * w_s[None, :]) * a_bf[:, None])
    # double rounding: an intermediate product narrowed to bf16 -- after the
    # weight scale it rounds the accumulator itself; after the activation
    # scale it only moves a rounding across an exact power-of-two multiply
    mid = synth.bf16_bits_to_f32(oracle.bf16_rne(f * w_s[None, :]))
    faults["double_rounding"] = oracle.bf16_rne(mid * a_s[:, None])
    mid = synth.bf16_bits_to_f32(oracle.bf16_rne(f * a_s[:, None]))
    faults["double_rounding_after_a_scale"] = oracle.bf16_rne(mid * w_s[None, :])
    # output truncation: fp32 -> bf16 by dropping the low half
    u = ((f * w_s[None, :]) * a_s[:, None]).astype(np.float32)
    faults["output_truncation"] = (u.view(np.uint32) >> 16).astype(np.uint16)
    # multiplication order: a_scale first (commutes exactly under pow2 w_scale)
    faults["multiplication_order"] = oracle.bf16_rne((f * a_s[:, None]) * w_s[None, :])
    # fused ordering: the two scales pre-multiplied into one factor
    faults["fused_scales"] = oracle.bf16_rne(f * (a_s[:, None] * w_s[None, :]))
    return ref, faults


def test_planted_epilogue_faults(small):
    """Power check: the faults that the power-of-two condition does not remove
    change some outputs by exactly one bf16 spacing and are caught by the
    0-ULP compare.  The multiplication-order fault and a narrowing placed
    after the activation scale are provably identical under power-of-two
    weight scales (a power-of-two multiply commutes with rounding), and so are
    pre-multiplied scales while the accumulator is exact in fp32
    (|acc| < 2^24), as here."""
    a_q, w_q, a_s, w_s = small
    _, acc = oracle.w8a8_pow2(a_q, w_q, a_s, w_s)
    assert np.abs(acc).max() < 2 ** 24
    ref, faults = _epilogue_variants(acc, a_s, w_s)
    for name in ("scale_precision", "double_rounding", "output_truncation"):
        diff = faults[name].astype(np.int32) - ref.astype(np.int32)
        assert np.any(diff != 0), name
        # bf16 patterns of one sign are ordered like integers: one spacing
        same_sign = (faults[name] >> 15) == (ref >> 15)
        assert np.abs(diff[same_sign]).max() == 1, name
    for name in ("multiplication_order", "fused_scales", "double_rounding_after_a_scale"):
        assert np.array_equal(faults[name], ref), name
