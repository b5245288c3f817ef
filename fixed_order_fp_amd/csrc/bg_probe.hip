// bg_probe.hip -- one matrix instruction per wavefront on crafted tiles: the
// black-box instrument for reconstructing how an instruction sums its
// products ("Taming Bitwise Behavior", section 4: place values, read the
// output; the emulator README's block-FMA model is one candidate answer).
//
// Operand placement (the same one the GEMM kernels use):
//   32x32x16 bf16: lane l holds A row (l % 32), k = 8*(l / 32) + i, i = 0..7;
//                  B likewise with n for m.  D: lane l, element e holds
//                  (m, n) = (8*(e/4) + 4*(l/32) + e%4, l % 32).
//   16x16x32 bf16: lane l holds A row (l % 16), k = 8*(l / 16) + i;
//                  D: lane l, element e holds (4*(l/16) + e, l % 16).
//   32x32x32 i8:   lane l holds A row (l % 32), k = 16*(l / 32) + i, i = 0..15.
//   16x16x64 i8:   lane l holds A row (l % 16), k = 16*(l / 16) + i.
#include "bg_internal.h"

namespace bg {

__global__ __launch_bounds__(64) void probe_f32_32x32x16_bf16(const uint16_t* A, const uint16_t* B,
                                                              const float* C, float* D)
{
    const int64_t c = blockIdx.x;
    const int l = threadIdx.x;
    const uint16_t* a = A + c * 32 * 16 + (l % 32) * 16 + 8 * (l / 32);
    const uint16_t* b = B + c * 32 * 16 + (l % 32) * 16 + 8 * (l / 32);
    bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)a);
    bf16x8 bv = __builtin_bit_cast(bf16x8, *(const u32x4*)b);
    f32x16 acc;
    for (int e = 0; e < 16; e++) {
        int m = 8 * (e / 4) + 4 * (l / 32) + e % 4, n = l % 32;
        acc[e] = C[c * 1024 + m * 32 + n];
    }
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
    for (int e = 0; e < 16; e++) {
        int m = 8 * (e / 4) + 4 * (l / 32) + e % 4, n = l % 32;
        D[c * 1024 + m * 32 + n] = acc[e];
    }
}

__global__ __launch_bounds__(64) void probe_f32_16x16x32_bf16(const uint16_t* A, const uint16_t* B,
                                                              const float* C, float* D)
{
    const int64_t c = blockIdx.x;
    const int l = threadIdx.x;
    const uint16_t* a = A + c * 16 * 32 + (l % 16) * 32 + 8 * (l / 16);
    const uint16_t* b = B + c * 16 * 32 + (l % 16) * 32 + 8 * (l / 16);
    bf16x8 av = __builtin_bit_cast(bf16x8, *(const u32x4*)a);
    bf16x8 bv = __builtin_bit_cast(bf16x8, *(const u32x4*)b);
    f32x4 acc;
    for (int e = 0; e < 4; e++) acc[e] = C[c * 256 + (4 * (l / 16) + e) * 16 + l % 16];
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
    for (int e = 0; e < 4; e++) D[c * 256 + (4 * (l / 16) + e) * 16 + l % 16] = acc[e];
}

__global__ __launch_bounds__(64) void probe_i32_32x32x32_i8(const int8_t* A, const int8_t* B,
                                                            const int32_t* C, int32_t* D)
{
    const int64_t c = blockIdx.x;
    const int l = threadIdx.x;
    i32x4 av = *(const i32x4*)(A + c * 32 * 32 + (l % 32) * 32 + 16 * (l / 32));
    i32x4 bv = *(const i32x4*)(B + c * 32 * 32 + (l % 32) * 32 + 16 * (l / 32));
    i32x16 acc;
    for (int e = 0; e < 16; e++) {
        int m = 8 * (e / 4) + 4 * (l / 32) + e % 4, n = l % 32;
        acc[e] = C[c * 1024 + m * 32 + n];
    }
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, acc, 0, 0, 0);
    for (int e = 0; e < 16; e++) {
        int m = 8 * (e / 4) + 4 * (l / 32) + e % 4, n = l % 32;
        D[c * 1024 + m * 32 + n] = acc[e];
    }
}

__global__ __launch_bounds__(64) void probe_i32_16x16x64_i8(const int8_t* A, const int8_t* B,
                                                            const int32_t* C, int32_t* D)
{
    const int64_t c = blockIdx.x;
    const int l = threadIdx.x;
    i32x4 av = *(const i32x4*)(A + c * 16 * 64 + (l % 16) * 64 + 16 * (l / 16));
    i32x4 bv = *(const i32x4*)(B + c * 16 * 64 + (l % 16) * 64 + 16 * (l / 16));
    i32x4 acc;
    for (int e = 0; e < 4; e++) acc[e] = C[c * 256 + (4 * (l / 16) + e) * 16 + l % 16];
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
    for (int e = 0; e < 4; e++) D[c * 256 + (4 * (l / 16) + e) * 16 + l % 16] = acc[e];
}

hipError_t launch_probe(int mfma, int64_t n_cases, const void* A, const void* B, const void* C,
                        void* D, hipStream_t stream)
{
    if (n_cases <= 0) return hipSuccess;
    dim3 grid((unsigned)n_cases), block(64);
    switch (mfma) {
    case BG_MFMA_F32_32X32X16_BF16:
        hipLaunchKernelGGL(probe_f32_32x32x16_bf16, grid, block, 0, stream, (const uint16_t*)A,
                           (const uint16_t*)B, (const float*)C, (float*)D);
        break;
    case BG_MFMA_F32_16X16X32_BF16:
        hipLaunchKernelGGL(probe_f32_16x16x32_bf16, grid, block, 0, stream, (const uint16_t*)A,
                           (const uint16_t*)B, (const float*)C, (float*)D);
        break;
    case BG_MFMA_I32_32X32X32_I8:
        hipLaunchKernelGGL(probe_i32_32x32x32_i8, grid, block, 0, stream, (const int8_t*)A,
                           (const int8_t*)B, (const int32_t*)C, (int32_t*)D);
        break;
    case BG_MFMA_I32_16X16X64_I8:
        hipLaunchKernelGGL(probe_i32_16x16x64_i8, grid, block, 0, stream, (const int8_t*)A,
                           (const int8_t*)B, (const int32_t*)C, (int32_t*)D);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace bg
