"""Seeded synthetic inputs shared by the GPU path's tests, the oracle's tests
and the bench.

This module holds none of the method's arithmetic: it draws numbers and
converts them to the storage types with library routines (numpy's float64 ->
float32 cast, torch's CPU float32 -> bfloat16 cast, numpy's rint), so that both
sides receive identical input bytes.

Recipe (every draw in row-major order of the full array):
  * N(mu, sigma) is drawn in float64 with numpy.random.default_rng(seed), cast
    to float32 (round to nearest), then to bfloat16 (round to nearest even).
  * The first operand of workload c uses seed 1000 + c, the second 2000 + c,
    the W8A8 weight-scale exponents 3005.
  * Exponent-spread draws (random sign, exponent uniform over a range,
    random significand) stand beside the ordinary ones because narrow
    exponents hide a regrouping ("Taming Bitwise Behavior", appendix E,
    validation method).
"""
import numpy as np

# ----------------------------------------------------------------------------
# storage conversions (library routines only)
# ----------------------------------------------------------------------------


def f32_to_bf16_bits(x):
    """float32 array -> bfloat16 bit patterns (uint16), via torch's CPU cast."""
    import torch
    x = np.asarray(x, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x).reshape(-1))
    h = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    return h.reshape(x.shape)


def bf16_bits_to_f32(h):
    """bfloat16 bit patterns -> float32 (exact: the low 16 bits are zero)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------


def f32_normal(seed, shape, mu=0.0, sigma=1.0):
    rng = np.random.default_rng(seed)
    return rng.normal(mu, sigma, size=shape).astype(np.float32)


def bf16_normal(seed, shape, mu=0.0, sigma=1.0):
    return f32_to_bf16_bits(f32_normal(seed, shape, mu, sigma))


def bf16_uniform_int(seed, shape, lo, hi):
    """bf16 whose values are integers uniform in [lo, hi] (exact in bf16 for
    |v| <= 256)."""
    rng = np.random.default_rng(seed)
    v = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return f32_to_bf16_bits(v)


def bf16_spread(seed, shape, emin=-20, emax=20):
    """bf16 bit patterns with random sign, unbiased exponent uniform in
    [emin, emax] and random 7-bit fraction."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=shape).astype(np.uint16) << 15
    exp = (rng.integers(emin, emax + 1, size=shape) + 127).astype(np.uint16) << 7
    frac = rng.integers(0, 128, size=shape).astype(np.uint16)
    return (sign | exp | frac).astype(np.uint16)


def f32_spread(seed, shape, emin=-20, emax=20):
    """float32 with random sign, exponent uniform in [emin, emax], random
    23-bit fraction."""
    rng = np.random.default_rng(seed)
    sign = rng.integers(0, 2, size=shape).astype(np.uint32) << 31
    exp = (rng.integers(emin, emax + 1, size=shape) + 127).astype(np.uint32) << 23
    frac = rng.integers(0, 1 << 23, size=shape).astype(np.uint32)
    return (sign | exp | frac).view(np.float32)


def int8_uniform(seed, shape, lo=-127, hi=127):
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.int8)


def pow2_scales(seed, n, emin=5, emax=12):
    """w_scale[n] = 2^-e with e uniform in [emin, emax] (exact in float32)."""
    rng = np.random.default_rng(seed)
    e = rng.integers(emin, emax + 1, size=n)
    return np.ldexp(np.ones(n, dtype=np.float32), -e).astype(np.float32)


def quantize_per_token(x):
    """Per-token absmax int8 quantisation, as input preparation (both sides
    receive the resulting bytes): a_scale = fp32(absmax) / 127 in float32;
    q = clamp(rint_even(x / a_scale), -127, 127) in float32; an all-zero row
    gets scale 1 and q = 0."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    q = np.rint((x / scale[:, None]).astype(np.float32))
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, scale


# ----------------------------------------------------------------------------
# the workloads
# ----------------------------------------------------------------------------


def gemm_small(K=512, M=32, N=64):
    """Small bf16 GEMM, 32x64x512: A, B ~ N(0,1) -> bf16 (seeds 1001, 2001)."""
    return bf16_normal(1001, (M, K)), bf16_normal(2001, (N, K))


def gemm_small_int(K=16, M=32, N=64):
    """K=16 small-integer variant: entries uniform in {-4..4}."""
    return bf16_uniform_int(1001, (M, K), -4, 4), bf16_uniform_int(2001, (N, K), -4, 4)


def gemm_batch_sweep(M=4000, N=9728, K=2560):
    """Batch-invariance sweep: X [4000][2560] ~ N(0,1) (seed 1003), W [9728][2560]
    ~ N(0, 0.02) (seed 2003), both bf16.  X_M is the first M rows."""
    X = bf16_normal(1003, (4000, K))[:M]
    W = bf16_normal(2003, (N, K), 0.0, 0.02)
    return X, W


def gemm_splitk_sweep(M=256, N=2560, K=9728):
    """Split-K sweep: A [256][9728] ~ N(0,1), W [2560][9728] ~ N(0, 0.02), bf16
    (seeds 1004, 2004)."""
    return bf16_normal(1004, (M, K)), bf16_normal(2004, (N, K), 0.0, 0.02)


def reduce_rows_input(rows=16384, cols=8192):
    """Row reductions: X [16384][8192] float32 ~ N(0,1), seed 1002."""
    return f32_normal(1002, (rows, cols))


def reduce_cols_input(rows=8192, cols=4096):
    """Column sum: Y [8192][4096] bf16 ~ N(0, 0.1), seed 2002."""
    return bf16_normal(2002, (rows, cols), 0.0, 0.1)


def w8a8_input(M=1024, N=6144, K=2048):
    """W8A8: activations N(0,1) [M][K] (seed 1005) quantised per token; weights
    int8 uniform in [-127, 127] [N][K] (seed 2005); weight scales 2^-e, e in
    [5, 12] (seed 3005)."""
    x = f32_normal(1005, (M, K))
    a_q, a_scale = quantize_per_token(x)
    w_q = int8_uniform(2005, (N, K))
    w_scale = pow2_scales(3005, N)
    return a_q, w_q, a_scale, w_scale
