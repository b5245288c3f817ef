// bg_ozaki.hip -- Ozaki-scheme GEMM on the int8 MFMA path (gfx950).
//
// "GPU Mechanism", the exact-GEMM paragraph and intervention (a) (ExactGEMM):
// each operand row is scaled by a power of two taken from frexp and cut into
// four signed 7-bit pieces; an integer GEMM multiplies the pieces exactly;
// the piece products are summed in fp64 in a set order and rounded once.  An
// integer sum is the same whatever order its terms arrive in, so neither the
// tile, the CU count nor anything else that moves a floating-point sum can
// reach the result.
//
//   slicing (one workgroup per row): e = frexp exponent of max |x| (0 for a
//     zero row); r = x * 2^-e in fp64 (exact, |r| < 1); for s = 0..3:
//     r = 128 r, q_s = trunc(r) in [-127, 127], r = r - q_s (all exact).
//     Slices go to [4][rows][Kp] int8 (Kp = K rounded up to 16, zero padded).
//   products: one int8 GEMM of the stacked slices, [4M][Kp] x [4N][Kp]^T,
//     into int32 [4M][4N] (the pipelined W8A8 kernel, accumulators only):
//     acc[sM + m][tN + n] = sum_k qA_s[m][k] qB_t[n][k].
//   recombination (one thread per output): v = sum over pairs of
//     acc_st 2^(-7 (s + t + 2)) in fp64, in the order s + t = 6, 5, ..., 0
//     (least significant first), s ascending within a level; v = v 2^(eA + eB);
//     one rounding to fp32 or bf16 (nearest even).
#include "bg_internal.h"

namespace bg {
namespace ozaki_impl {

template <bool IN_BF16>
__device__ __forceinline__ float elem(const void* X, int64_t i)
{
    if constexpr (IN_BF16) return bf16_to_f32(((const uint16_t*)X)[i]);
    else return ((const float*)X)[i];
}

template <bool IN_BF16>
__global__ __launch_bounds__(256) void ozaki_slice_kernel(const void* __restrict__ X, int64_t ldx, int64_t rows,
                                                          int64_t K, int64_t Kp, int8_t* __restrict__ Q,
                                                          int* __restrict__ E)
{
    __shared__ float wmax[4];
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    float amax = 0.0f;  // a maximum is exact in any order
    for (int64_t k = t; k < K; k += 256) amax = fmaxf(amax, fabsf(elem<IN_BF16>(X, r * ldx + k)));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax in [2^(e-1), 2^e)
    if (t == 0) E[r] = e;
    // four consecutive k per thread (Kp is a multiple of 16), each slice's
    // four codes written as one 32-bit word
    for (int64_t k0 = 4 * (int64_t)t; k0 < Kp; k0 += 1024) {
        uint32_t packed[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int64_t k = k0 + u;
            double v = k < K ? ldexp((double)elem<IN_BF16>(X, r * ldx + k), -e) : 0.0;
#pragma unroll
            for (int s = 0; s < 4; s++) {
                v = v * 128.0;
                const double q = trunc(v);
                packed[s] |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * u);
                v = v - q;
            }
        }
#pragma unroll
        for (int s = 0; s < 4; s++) *(uint32_t*)(Q + ((int64_t)s * rows + r) * Kp + k0) = packed[s];
    }
}

// fp64 -> bf16 bits, one rounding to nearest even (no pass through fp32)
__device__ __forceinline__ uint16_t bf16_from_f64(double v)
{
    if (v != v) return 0x7fc0;
    const uint16_t sign = __builtin_signbit(v) ? 0x8000 : 0;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);              // a in [2^(e-1), 2^e)
    int ue = e - 8;                  // bf16 keeps 8 significant bits
    if (ue < -133) ue = -133;        // subnormal spacing 2^-133
    const double y = ldexp(rint(ldexp(a, -ue)), ue);
    if (y >= 0x1p128) return sign | 0x7f80;
    const float f = (float)y;        // exact: at most 8 significant bits
    return (uint16_t)(sign | ((__float_as_uint(f) >> 16) & 0x7fff));
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void ozaki_combine_kernel(const int32_t* __restrict__ acc, int64_t M, int64_t N,
                                                            const int* __restrict__ EA, const int* __restrict__ EB,
                                                            void* __restrict__ C, int64_t ldc)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx % N;
    const int64_t ld = 4 * N;
    double v = 0.0;
#pragma unroll
    for (int lev = 6; lev >= 0; lev--)
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int t = lev - s;
            if (t < 0 || t > 3) continue;
            // each product is read once, by whole lines: a streaming load
            v = v + ldexp((double)__builtin_nontemporal_load(&acc[(s * M + m) * ld + t * N + n]), -7 * (lev + 2));
        }
    v = ldexp(v, EA[m] + EB[n]);
    if constexpr (OUT_BF16) ((uint16_t*)C)[m * ldc + n] = bf16_from_f64(v);
    else ((float*)C)[m * ldc + n] = (float)v;  // one rounding, nearest even
}

}  // namespace ozaki_impl

using namespace ozaki_impl;

hipError_t launch_ozaki(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, bool in_bf16, const void* A, int64_t lda,
                        const void* B, int64_t ldb, bool out_bf16, void* C, int64_t ldc, const OzakiWs& w,
                        hipStream_t stream)
{
    if (in_bf16) {
        hipLaunchKernelGGL(ozaki_slice_kernel<true>, dim3((unsigned)M), dim3(256), 0, stream, A, lda, M, K, w.Kp,
                           w.qa, w.ea);
        hipLaunchKernelGGL(ozaki_slice_kernel<true>, dim3((unsigned)N), dim3(256), 0, stream, B, ldb, N, K, w.Kp,
                           w.qb, w.eb);
    } else {
        hipLaunchKernelGGL(ozaki_slice_kernel<false>, dim3((unsigned)M), dim3(256), 0, stream, A, lda, M, K, w.Kp,
                           w.qa, w.ea);
        hipLaunchKernelGGL(ozaki_slice_kernel<false>, dim3((unsigned)N), dim3(256), 0, stream, B, ldb, N, K, w.Kp,
                           w.qb, w.eb);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_w8a8(p, 4 * M, 4 * N, w.Kp, w.qa, w.Kp, w.qb, w.Kp, nullptr, nullptr, nullptr, 0, w.acc, 4 * N, stream);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((M * N + 255) / 256));
    if (out_bf16)
        hipLaunchKernelGGL(ozaki_combine_kernel<true>, grid, dim3(256), 0, stream, w.acc, M, N, w.ea, w.eb, C, ldc);
    else
        hipLaunchKernelGGL(ozaki_combine_kernel<false>, grid, dim3(256), 0, stream, w.acc, M, N, w.ea, w.eb, C, ldc);
    return hipGetLastError();
}

}  // namespace bg
