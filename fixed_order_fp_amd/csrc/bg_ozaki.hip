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
//     Slices go to [rows][4][Kp] int8, row 4r + s holding slice s of row r
//     (Kp = K rounded up to 16, zero padded).
//   products and recombination in one launch: the int8 GEMM of the stacked
//     slices, [4M][Kp] x [4N][Kp]^T on the pipelined W8A8 kernel, whose
//     stacked output (4m + s, 4n + t) is acc_st = sum_k qA_s[m][k] qB_t[n][k];
//     its epilogue finds all sixteen acc_st of an output in one 32x32 block
//     and sums acc_st 2^(-7 (s + t + 2)) in fp64 in the order s + t = 6, 5,
//     ..., 0 (least significant first), s ascending within a level; then
//     v = v 2^(eA + eB) and one rounding to fp32 or bf16 (nearest even).
//     The products are never written out.
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
        for (int s = 0; s < 4; s++) *(uint32_t*)(Q + (4 * r + s) * Kp + k0) = packed[s];
    }
}

// The same slicing for rows that can be read 16 bytes at a time (16-byte
// aligned rows, K and ldx multiples of the elements per 16 bytes) and that
// fit in registers (at most 8 chunks of 16 bytes per thread): the row is read
// once, its maximum taken from the registers, and each chunk's four slices
// written as 4 x (8 or 4) bytes.  Chunks of the padding [K, Kp) hold zeros.
template <bool IN_BF16>
__global__ __launch_bounds__(256) void ozaki_slice_vec_kernel(const void* __restrict__ X, int64_t ldx, int64_t K,
                                                              int64_t Kp, int8_t* __restrict__ Q,
                                                              int* __restrict__ E)
{
    constexpr int EPC = IN_BF16 ? 8 : 4;  // elements per 16-byte chunk
    constexpr int RMAX = 8;
    __shared__ float wmax[4];
    const int64_t r = blockIdx.x;
    const int t = threadIdx.x;
    const int n_load = (int)(K / EPC), n_all = (int)((Kp + EPC - 1) / EPC);
    const char* row = (const char*)X + r * ldx * (IN_BF16 ? 2 : 4);
    u32x4 v[RMAX];
#pragma unroll
    for (int i = 0; i < RMAX; i++) {
        const int c = t + 256 * i;
        v[i] = c < n_load ? *(const u32x4*)(row + 16 * (int64_t)c) : u32x4{0u, 0u, 0u, 0u};
    }
    auto val = [&](const u32x4& w, int j) -> float {
        if constexpr (IN_BF16) return __uint_as_float(j & 1 ? (w[j / 2] & 0xffff0000u) : (w[j / 2] << 16));
        else return __uint_as_float(w[j]);
    };
    float amax = 0.0f;  // a maximum is exact in any order
#pragma unroll
    for (int i = 0; i < RMAX; i++)
#pragma unroll
        for (int j = 0; j < EPC; j++) amax = fmaxf(amax, fabsf(val(v[i], j)));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((t & 63) == 0) wmax[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax in [2^(e-1), 2^e)
    if (t == 0) E[r] = e;
#pragma unroll
    for (int i = 0; i < RMAX; i++) {
        const int c = t + 256 * i;
        if (c >= n_all) break;
        uint32_t packed[4][EPC / 4] = {};
#pragma unroll
        for (int j = 0; j < EPC; j++) {
            double d = ldexp((double)val(v[i], j), -e);  // zero past K: the chunk was not loaded
#pragma unroll
            for (int s4 = 0; s4 < 4; s4++) {
                d = d * 128.0;
                const double q = trunc(d);
                packed[s4][j / 4] |= (uint32_t)(uint8_t)(int8_t)(int)q << (8 * (j % 4));
                d = d - q;
            }
        }
#pragma unroll
        for (int s4 = 0; s4 < 4; s4++) {
            int8_t* dst = Q + (4 * r + s4) * Kp + (int64_t)c * EPC;
            if constexpr (EPC == 8) *(uint2*)dst = uint2{packed[s4][0], packed[s4][1]};
            else *(uint32_t*)dst = packed[s4][0];
        }
    }
}

}  // namespace ozaki_impl

using namespace ozaki_impl;

hipError_t launch_ozaki(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, bool in_bf16, const void* A, int64_t lda,
                        const void* B, int64_t ldb, bool out_bf16, void* C, int64_t ldc, const OzakiWs& w,
                        hipStream_t stream)
{
    // one operand: the vector kernel where its rows allow, else the plain one
    auto slice = [&](const void* X, int64_t ldx, int64_t rows, int8_t* q, int* ex) {
        const int64_t epc = in_bf16 ? 8 : 4;
        const bool vec = ((uintptr_t)X % 16) == 0 && ldx % epc == 0 && K % epc == 0 && (w.Kp + epc - 1) / epc <= 8 * 256;
        if (vec && in_bf16)
            hipLaunchKernelGGL(ozaki_slice_vec_kernel<true>, dim3((unsigned)rows), dim3(256), 0, stream, X, ldx, K, w.Kp,
                               q, ex);
        else if (vec)
            hipLaunchKernelGGL(ozaki_slice_vec_kernel<false>, dim3((unsigned)rows), dim3(256), 0, stream, X, ldx, K,
                               w.Kp, q, ex);
        else if (in_bf16)
            hipLaunchKernelGGL(ozaki_slice_kernel<true>, dim3((unsigned)rows), dim3(256), 0, stream, X, ldx, rows, K,
                               w.Kp, q, ex);
        else
            hipLaunchKernelGGL(ozaki_slice_kernel<false>, dim3((unsigned)rows), dim3(256), 0, stream, X, ldx, rows, K,
                               w.Kp, q, ex);
    };
    slice(A, lda, M, w.qa, w.ea);
    slice(B, ldb, N, w.qb, w.eb);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_w8a8_ozaki(p, 4 * M, 4 * N, w.Kp, w.qa, w.qb, w.ea, w.eb, out_bf16, C, ldc, stream);
}

}  // namespace bg
