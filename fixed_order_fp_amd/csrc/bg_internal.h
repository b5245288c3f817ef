// bg_internal.h -- shared device types and host launcher declarations of
// libbitgemm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bitgemm.h"

namespace bg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest, ties to even; a NaN becomes the quiet
// NaN 0x7fc0 carrying the input's sign.
__device__ __forceinline__ uint16_t bf16_rne(float x)
{
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> two bf16 packed in one word (x0 in the low half), with gfx950's
// conversion instruction: round to nearest, ties to even, bit-identical to
// bf16_rne for every non-NaN input (checked over all 2^32 patterns on MI355X).
// The instruction keeps a NaN's payload; the NaN halves are then replaced by
// 0x7fc0 under their own sign, which is what bf16_rne gives.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float x0, float x1)
{
    const f32x2_t f = {x0, x1};
    const uint32_t p = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    const uint32_t m = (x0 != x0 ? 0x00007fffu : 0u) | (x1 != x1 ? 0x7fff0000u : 0u);
    return (p & ~m) | (0x7fc07fc0u & m);
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

// ---- plans handed from the C ABI layer to the launchers -------------------
struct Cuts {
    int64_t c[BG_MAX_SPLIT + 1];
};

// Reductions of the fp32 C tile in the GEMM epilogue: one fp32 leaf node per
// 32 consecutive rows (column axis) or columns (row axis) of C and per output,
// written as ws[leaf][n_out]; NULL pointers skip that output.
struct RedArgs {
    float* ws_sum;
    float* ws_sq;
    int64_t n_out;  // N for the column axis, M for the row axis
    int fused;      // sum of squares by fma
};

struct GemmPlan {
    int S;           // splits
    Cuts cuts;       // cut points, cuts.c[0] = 0, cuts.c[S] = K
    int mfma;        // bg_mfma
    bool out_bf16;   // rounding point target
    int bm, bn, bk;  // schedule
    int waves_m, waves_n;
    int direct;      // 1: operand tiles copied global -> LDS directly; 2: pipelined
    int stages;      // k tiles in LDS (pipelined path)
    int group_m;     // tile rows per group of the workgroup walk
    int bm2, bn2;    // the last split's tile (pipelined path, S > 1); 0 = none
    int waves_m2, waves_n2, stages2;
    bool last_first; // dispatch the last split's workgroups before the others
    bool atomic;     // free-order twin: splits added into a zeroed fp32 C with atomics
    int red;         // fused reduction of C: 0 none, 1 column leaves, 2 row leaves
    RedArgs red_args;
};

hipError_t launch_probe(int mfma, int64_t n_cases, const void* A, const void* B, const void* C,
                        void* D, hipStream_t stream);

hipError_t launch_gemm_bf16(const GemmPlan& p, int64_t M, int64_t N, int64_t K,
                            const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                            void* C, int64_t ldc, float* ws, hipStream_t stream);

struct W8A8Plan {
    int mfma;  // BG_MFMA_I32_32X32X32_I8 | BG_MFMA_I32_16X16X64_I8
    int bm, bn, waves_m, waves_n, group_m;
    int path;    // 1: direct-to-LDS double buffer; 2: pipelined (32x32x32 only)
    int stages;  // k tiles in LDS (pipelined path; 0 = the tile's default)
    bool free_epilogue;  // free-order twin (bench only): y = fp32(acc) * (a_scale * w_scale)
};

bool w8a8_has_tile(int mfma, int bm, int bn, int waves_m, int waves_n, int path, int stages);
hipError_t launch_w8a8(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y,
                       int64_t ldy, int32_t* acc_out, int64_t ld_acc, hipStream_t stream);

// Ozaki-scheme GEMM workspace: slices [4][M][Kp] and [4][N][Kp] int8, row
// exponents, the stacked int32 products [4M][4N].
struct OzakiWs {
    int64_t Kp;
    int8_t* qa;
    int8_t* qb;
    int* ea;
    int* eb;
};
// the Ozaki GEMM's products and recombination (stacked sizes M4 = 4 M, N4 =
// 4 N; slices interleaved as rows 4r + s); pipelined tiles listed in
// bg_w8a8.hip only
bool w8a8_ozaki_has_tile(const W8A8Plan& p);
hipError_t launch_w8a8_ozaki(const W8A8Plan& p, int64_t M4, int64_t N4, int64_t Kp, const int8_t* qa,
                             const int8_t* qb, const int* ea, const int* eb, bool out_bf16, void* C, int64_t ldc,
                             hipStream_t stream);
// Y == nullptr: the int32 accumulators only (pipelined tiles)
hipError_t launch_ozaki(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, bool in_bf16, const void* A, int64_t lda,
                        const void* B, int64_t ldb, bool out_bf16, void* C, int64_t ldc, const OzakiWs& w,
                        hipStream_t stream);

struct ReducePlan {
    int axis;          // BG_AXIS_ROW | BG_AXIS_COL
    bool bf16;         // input type
    bool fused;        // q = fma(x, x, q)
    int leaves_per_wg; // column axis: leaves one workgroup folds (4, 8, 16, 32)
    int cols_per_lane; // column axis, bf16 input: 4 or 8
    bool col_full;     // column axis: one pass, a workgroup per strip over every row
};

int64_t reduce_row_blocks(int64_t cols);
int64_t reduce_col_blocks(int64_t rows, int lpw);
hipError_t launch_reduce(const ReducePlan& p, int64_t rows, int64_t cols, const void* X, int64_t ldx,
                         float* out_sum, float* out_sq, float* ws, hipStream_t stream);
hipError_t launch_reduce_free(int axis, bool bf16, int64_t rows, int64_t cols, const void* X, int64_t ldx,
                              float* out_sum, float* out_sq, int n_cu, hipStream_t stream);

// Balanced tree over leaf nodes ws[leaf][n_out] (n_leaf <= 1024) per output.
hipError_t launch_leaf_tree(const float* ws_sum, const float* ws_sq, int64_t n_out, int n_leaf, float* out_sum,
                            float* out_sq, hipStream_t stream);

hipError_t launch_quantize_rows(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q, int64_t ldq,
                                float* scale, bool vec, hipStream_t stream);
hipError_t launch_requantize_pow2(int64_t N, int64_t K, const int8_t* W, int64_t ldw, const float* w_scale,
                                  int mode, int8_t* W2, int64_t ldw2, float* w_scale2, bool vec,
                                  hipStream_t stream);

// which tile shapes the GEMM kernel is instantiated for
hipError_t launch_zero_rows(float* C, int64_t M, int64_t N, int64_t ldc, hipStream_t stream);
bool gemm_bf16_has_tile(int mfma, int bm, int bn, int bk, int waves_m, int waves_n, int direct, int stages);
// a compiled (other splits, last split) pair of pipelined tiles; stages == 0
// takes the first compiled pair of the two shapes
bool gemm_bf16_has_dual_tile(int bm, int bn, int bk, int waves_m, int waves_n, int stages, int bm2, int bn2,
                             int waves_m2, int waves_n2, int stages2);
// tiles built with the fused reductions (pipelined path, S = 1)
bool gemm_bf16_red_has_tile(int bm, int bn, int bk, int waves_m, int waves_n, int stages);

// The 64-deep pipelined tiles address each copy by a 32-bit byte offset from
// the tile's first row: (rows - 1) x leading dimension x 2 bytes, plus a
// 128-byte row piece, must stay below 2^32.
inline bool pipe_offsets_fit(int64_t bm, int64_t bn, int64_t lda, int64_t ldb)
{
    const int64_t lim = (int64_t)1 << 32;
    return (bm - 1) * lda * 2 + 128 < lim && (bn - 1) * ldb * 2 + 128 < lim;
}
// the same for the two-stage W8A8 tiles (int8 operands: one byte per element)
inline bool i8_offsets_fit(int64_t bm, int64_t bn, int64_t lda, int64_t ldw)
{
    const int64_t lim = (int64_t)1 << 32;
    return (bm - 1) * lda + 128 < lim && (bn - 1) * ldw + 128 < lim;
}
hipError_t launch_gemm_bf16_reduce(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                                   const uint16_t* B, int64_t ldb, void* C, int64_t ldc, hipStream_t stream);
hipError_t launch_gemm_bf16_two_chains(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                       const uint16_t* B, int64_t ldb, float* C, int64_t ldc, hipStream_t stream);

}  // namespace bg
