// bg_quant.hip -- int8 quantisation on either side of the W8A8 GEMM (gfx950).
//
// Activations, per token: a workgroup owns one row; pass 1 takes max |x| over
// the row (a maximum is exact, so the lanes may meet in any order), pass 2
// writes clamp(rint(x / scale), -127, 127) with scale = fp32(absmax) / 127
// (an all-zero row takes scale 1).  The row is read twice; the second read is
// served by L2 (one row is at most a few tens of KB).
//
// Weights ("Deterministic LLM Inference ... Power-of-Two INT8 Quantization
// Scales", section V: the int8 weights themselves are recomputed for the
// power-of-two scale; changing the scale alone would not do): per output row, s2 = 2^e with e = round(log2 s)
// (nearest in ratio) or ceil(log2 s); each weight becomes
// clamp(rint(fp32(q * s) / s2), -127, 127), the product rounded once and the
// division by a power of two exact (done as a multiplication by the exact
// reciprocal where that is a normal float).
//
// Divisions are IEEE (correctly rounded: hipcc's default for fp32 division),
// rint rounds ties to even, and a NaN quotient gives 0.
#include "bg_internal.h"

namespace bg {
namespace quant_impl {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int8_t clamp_code(float r)
{
    if (r != r) return 0;
    r = r > 127.0f ? 127.0f : r;
    r = r < -127.0f ? -127.0f : r;
    return (int8_t)(int)r;
}

__device__ __forceinline__ uint32_t pack4(int8_t a, int8_t b, int8_t c, int8_t d)
{
    return (uint32_t)(uint8_t)a | ((uint32_t)(uint8_t)b << 8) | ((uint32_t)(uint8_t)c << 16) |
           ((uint32_t)(uint8_t)d << 24);
}

// VEC: X 16-byte aligned rows of K % 4 == 0 floats, Q rows 4-byte aligned
template <bool VEC>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float* __restrict__ X, int64_t ldx, int64_t K,
                                                            int8_t* __restrict__ Q, int64_t ldq,
                                                            float* __restrict__ scale)
{
    __shared__ float wmax[4];
    const int64_t m = blockIdx.x;
    const float* x = X + m * ldx;
    int8_t* q = Q + m * ldq;
    const int t = threadIdx.x;

    // rows of up to 1024 R floats stay in registers between the two passes
    // (one read of the row, streaming); longer rows are read twice, the
    // second time from L2
    constexpr int R = 8;
    const bool in_regs = VEC && K <= 1024 * R;
    f32x4_t reg[R];
    float amax = 0.0f;  // fmaxf ignores a NaN operand, as a "greater than" scan does
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < R; i++) {
            const int64_t k = 4 * (int64_t)t + 1024 * i;
            reg[i] = k < K ? __builtin_nontemporal_load((const f32x4_t*)(x + k)) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(reg[i].x), fabsf(reg[i].y)), fmaxf(fabsf(reg[i].z), fabsf(reg[i].w))));
        }
    } else if constexpr (VEC) {
        for (int64_t k = 4 * (int64_t)t; k < K; k += 1024) {
            const f32x4_t v = *(const f32x4_t*)(x + k);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        }
    } else {
        for (int64_t k = t; k < K; k += 256) amax = fmaxf(amax, fabsf(x[k]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float s = amax > 0.0f ? amax / 127.0f : 1.0f;
    if (t == 0) scale[m] = s;

    if (in_regs) {
#pragma unroll
        for (int i = 0; i < R; i++) {
            const int64_t k = 4 * (int64_t)t + 1024 * i;
            if (k < K)
                *(uint32_t*)(q + k) = pack4(clamp_code(rintf(reg[i].x / s)), clamp_code(rintf(reg[i].y / s)),
                                            clamp_code(rintf(reg[i].z / s)), clamp_code(rintf(reg[i].w / s)));
        }
    } else if constexpr (VEC) {
        for (int64_t k = 4 * (int64_t)t; k < K; k += 1024) {
            const f32x4_t v = *(const f32x4_t*)(x + k);
            *(uint32_t*)(q + k) = pack4(clamp_code(rintf(v.x / s)), clamp_code(rintf(v.y / s)),
                                        clamp_code(rintf(v.z / s)), clamp_code(rintf(v.w / s)));
        }
    } else {
        for (int64_t k = t; k < K; k += 256) q[k] = clamp_code(rintf(x[k] / s));
    }
}

__device__ __forceinline__ float pow2_scale(float s, int mode)
{
    if (!(s > 0.0f) || __builtin_isinf(s)) return s;
    int ex;
    (void)frexpf(s, &ex);  // s in [2^(ex-1), 2^ex)
    int e;
    if (mode == BG_POW2_CEIL) {
        e = (s == ldexpf(1.0f, ex - 1)) ? ex - 1 : ex;
    } else {
        // log2 s rounds up exactly when s*s >= 2^(2 ex - 1) (s*s is exact in double)
        const double sq = (double)s * (double)s;
        e = (sq >= ldexp(1.0, 2 * ex - 1)) ? ex : ex - 1;
    }
    return ldexpf(1.0f, e);
}

// VEC: rows of K % 16 == 0 bytes, 16-byte aligned.  A workgroup takes two
// rows, 128 threads each.
template <bool VEC>
__global__ __launch_bounds__(256) void requantize_pow2_kernel(int64_t N, const int8_t* __restrict__ W, int64_t ldw,
                                                              int64_t K, const float* __restrict__ w_scale, int mode,
                                                              int8_t* __restrict__ W2, int64_t ldw2,
                                                              float* __restrict__ w_scale2)
{
    const int64_t n = (int64_t)blockIdx.x * 2 + (threadIdx.x >> 7);
    if (n >= N) return;
    const int8_t* w = W + n * ldw;
    int8_t* o = W2 + n * ldw2;
    const int t = threadIdx.x & 127;
    const float s = w_scale[n];
    const bool usable = s > 0.0f && !__builtin_isinf(s);
    const float s2 = pow2_scale(s, mode);
    if (t == 0) w_scale2[n] = s2;
    // dividing by 2^e is multiplying by 2^-e, a correctly rounded result of
    // the same exact value, whenever 2^-e is a normal float
    const bool by_mul = s2 >= 0x1p-126f && s2 <= 0x1p126f;
    const float inv = by_mul ? 1.0f / s2 : 0.0f;
    auto code = [&](int8_t v) -> int8_t {
        if (!usable) return v;
        const float p = (float)v * s;  // one rounding
        return clamp_code(rintf(by_mul ? p * inv : p / s2));
    };
    if constexpr (VEC) {
        for (int64_t k = 16 * (int64_t)t; k < K; k += 2048) {
            const u32x4 v = __builtin_nontemporal_load((const u32x4*)(w + k));
            u32x4 r;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t u = v[i];
                r[i] = pack4(code((int8_t)(u & 0xff)), code((int8_t)((u >> 8) & 0xff)),
                             code((int8_t)((u >> 16) & 0xff)), code((int8_t)(u >> 24)));
            }
            __builtin_nontemporal_store(r, (u32x4*)(o + k));
        }
    } else {
        for (int64_t k = t; k < K; k += 128) o[k] = code(w[k]);
    }
}

}  // namespace quant_impl

using namespace quant_impl;

hipError_t launch_quantize_rows(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q, int64_t ldq,
                                float* scale, bool vec, hipStream_t stream)
{
    dim3 grid((unsigned)M), block(256);
    if (vec)
        hipLaunchKernelGGL(quantize_rows_kernel<true>, grid, block, 0, stream, X, ldx, K, Q, ldq, scale);
    else
        hipLaunchKernelGGL(quantize_rows_kernel<false>, grid, block, 0, stream, X, ldx, K, Q, ldq, scale);
    return hipGetLastError();
}

hipError_t launch_requantize_pow2(int64_t N, int64_t K, const int8_t* W, int64_t ldw, const float* w_scale,
                                  int mode, int8_t* W2, int64_t ldw2, float* w_scale2, bool vec,
                                  hipStream_t stream)
{
    dim3 grid((unsigned)((N + 1) / 2)), block(256);
    if (vec)
        hipLaunchKernelGGL(requantize_pow2_kernel<true>, grid, block, 0, stream, N, W, ldw, K, w_scale, mode, W2,
                           ldw2, w_scale2);
    else
        hipLaunchKernelGGL(requantize_pow2_kernel<false>, grid, block, 0, stream, N, W, ldw, K, w_scale, mode, W2,
                           ldw2, w_scale2);
    return hipGetLastError();
}

}  // namespace bg
