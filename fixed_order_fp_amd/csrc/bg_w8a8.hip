// bg_w8a8.hip -- W8A8 GEMM with power-of-two weight scales for gfx950
// ("Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
// Quantization Scales", section II): Y = (A W^T) s_a s_w with int8 operands
// and exact int32 accumulation, so any tiling or order gives the same
// accumulator; the epilogue then fixes the one place where order matters:
//   f = fp32(acc) (round to nearest even), t = f * w_scale[n] (exact for a
//   power of two), u = t * a_scale[m] (one rounding), y = bf16_rne(u).
// No multiply-add is fused (built with -ffp-contract=off; the epilogue has no
// add at all).
//
// Data path as in the bf16 direct kernel: 128-byte k tiles (128 int8) of A
// and W copied global -> LDS with global_load_lds_dwordx4 under a row-XOR
// swizzle, double-buffered; v_mfma_i32_32x32x32_i8 or v_mfma_i32_16x16x64_i8
// with one 16-byte chunk per lane per instruction.
#include "bg_internal.h"

namespace bg {

namespace w8a8_impl {

constexpr int kChunk = 16;  // int8 per 16-byte chunk
constexpr int BK = 128;     // int8 per k tile
constexpr int CPR = BK / kChunk;

template <int INSTR>
struct I8Shape;
template <>
struct I8Shape<BG_MFMA_I32_32X32X32_I8> {
    static constexpr int M = 32, N = 32, K = 32, ACC = 16;
    typedef i32x16 acc_t;
};
template <>
struct I8Shape<BG_MFMA_I32_16X16X64_I8> {
    static constexpr int M = 16, N = 16, K = 64, ACC = 4;
    typedef i32x4 acc_t;
};

template <int INSTR>
__device__ __forceinline__ typename I8Shape<INSTR>::acc_t mfma_i8(i32x4 a, i32x4 b, typename I8Shape<INSTR>::acc_t c)
{
    if constexpr (INSTR == BG_MFMA_I32_32X32X32_I8)
        return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void lds_copy16(const void* src, u32x4* lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

__device__ __forceinline__ int slot(int row, int kc) { return row * CPR + (kc ^ (row & 7)); }

// 16 int8 at k .. k+15 of a row, zero beyond k_end.
__device__ __forceinline__ u32x4 load_chunk_i8(const int8_t* row_ptr, int64_t k, int64_t k_end)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k >= k_end) return v;
    if (k + kChunk <= k_end) return *(const u32x4*)(row_ptr + k);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    for (int j = 0; j < kChunk; j++)
        if (k + j < k_end) w[j / 4] |= (uint32_t)(uint8_t)row_ptr[k + j] << (8 * (j % 4));
    v[0] = w[0], v[1] = w[1], v[2] = w[2], v[3] = w[3];
    return v;
}

__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int group_m, int& tm, int& tn)
{
    const int T = tiles_m * tiles_n;
    const int q = T / 8, r = T % 8;
    const int x = b % 8, j = b / 8;
    const int bb = x * q + (x < r ? x : r) + j;
    const int per_group = group_m * tiles_n;
    const int g = bb / per_group;
    const int first_m = g * group_m;
    const int gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in = bb - g * per_group;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

template <int INSTR, int BM, int BN, int WM, int WN, bool ACC_OUT>
__global__ __launch_bounds__(64 * WM * WN) void w8a8_kernel(
    const int8_t* __restrict__ A, int64_t lda, const int8_t* __restrict__ W, int64_t ldw,
    const float* __restrict__ a_scale, const float* __restrict__ w_scale, uint16_t* __restrict__ Y, int64_t ldy,
    int32_t* __restrict__ acc_out, int64_t ld_acc, int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n,
    int group_m)
{
    typedef I8Shape<INSTR> S;
    constexpr int NW = WM * WN, NT = 64 * NW;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / S::M, TN = WTN / S::N;
    constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
    constexpr int A_PER_T = A_CH / NT, B_PER_T = B_CH / NT;
    static_assert(A_CH % NT == 0 && B_CH % NT == 0, "tile must split evenly over the waves");

    __shared__ u32x4 lds_a[2][A_CH];
    __shared__ u32x4 lds_b[2][B_CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
    const int n_full = (int)(K / BK);
    const int n_turns = (int)((K + BK - 1) / BK);

    const int8_t* a_src[A_PER_T];
    const int8_t* b_src[B_PER_T];
    int a_kc[A_PER_T], b_kc[B_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; i++) {
        const int c = i * NT + wave * 64 + lane;
        const int row = c / CPR;
        a_kc[i] = (c % CPR) ^ (row & 7);
        int64_t gm = m0 + row;
        gm = gm < M ? gm : M - 1;
        a_src[i] = A + gm * lda + a_kc[i] * kChunk;
    }
#pragma unroll
    for (int i = 0; i < B_PER_T; i++) {
        const int c = i * NT + wave * 64 + lane;
        const int row = c / CPR;
        b_kc[i] = (c % CPR) ^ (row & 7);
        int64_t gn = n0 + row;
        gn = gn < N ? gn : N - 1;
        b_src[i] = W + gn * ldw + b_kc[i] * kChunk;
    }

    typename S::acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < S::ACC; e++) acc[i][j][e] = 0;

    auto issue = [&](int turn, int stage) {
        const int64_t kb = (int64_t)turn * BK;
        if (turn < n_full) {
#pragma unroll
            for (int i = 0; i < A_PER_T; i++) lds_copy16(a_src[i] + kb, &lds_a[stage][i * NT + wave * 64]);
#pragma unroll
            for (int i = 0; i < B_PER_T; i++) lds_copy16(b_src[i] + kb, &lds_b[stage][i * NT + wave * 64]);
        } else {
#pragma unroll
            for (int i = 0; i < A_PER_T; i++)
                lds_a[stage][i * NT + wave * 64 + lane] = load_chunk_i8(a_src[i] - a_kc[i] * kChunk, kb + a_kc[i] * kChunk, K);
#pragma unroll
            for (int i = 0; i < B_PER_T; i++)
                lds_b[stage][i * NT + wave * 64 + lane] = load_chunk_i8(b_src[i] - b_kc[i] * kChunk, kb + b_kc[i] * kChunk, K);
        }
    };
    auto compute = [&](int stage) {
        const int r_in = lane % S::M;
        const int kc_in = lane / S::M;
#pragma unroll
        for (int ks = 0; ks < BK / S::K; ks++) {
            i32x4 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; i++)
                a[i] = __builtin_bit_cast(i32x4, lds_a[stage][slot(wm * WTM + i * S::M + r_in, ks * (S::K / kChunk) + kc_in)]);
#pragma unroll
            for (int j = 0; j < TN; j++)
                b[j] = __builtin_bit_cast(i32x4, lds_b[stage][slot(wn * WTN + j * S::N + r_in, ks * (S::K / kChunk) + kc_in)]);
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) acc[i][j] = mfma_i8<INSTR>(a[i], b[j], acc[i][j]);
        }
    };

    if (n_turns > 0) issue(0, 0);
    for (int t = 0; t < n_turns; t++) {
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
        if (t + 1 < n_turns) issue(t + 1, (t + 1) & 1);
        compute(t & 1);
    }

#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < S::ACC; e++) {
                int rm, cn;
                if constexpr (S::M == 32) {
                    rm = 8 * (e / 4) + 4 * (lane / 32) + (e % 4);
                    cn = lane % 32;
                } else {
                    rm = 4 * (lane / 16) + e;
                    cn = lane % 16;
                }
                const int64_t gm = m0 + wm * WTM + i * S::M + rm;
                const int64_t gn = n0 + wn * WTN + j * S::N + cn;
                if (gm < M && gn < N) {
                    const int32_t v = acc[i][j][e];
                    const float f = (float)v;          // v_cvt_f32_i32: round to nearest even
                    const float t = f * w_scale[gn];  // exact: a power of two
                    const float u = t * a_scale[gm];  // the one rounding
                    Y[gm * ldy + gn] = bf16_rne(u);
                    if constexpr (ACC_OUT) acc_out[gm * ld_acc + gn] = v;
                }
            }
}

template <int INSTR, int BM, int BN, int WM, int WN>
hipError_t launch(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                  const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y, int64_t ldy,
                  int32_t* acc_out, int64_t ld_acc, hipStream_t stream)
{
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int group_m = p.group_m > 0 ? p.group_m : 8;
    dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
    if (acc_out)
        hipLaunchKernelGGL((w8a8_kernel<INSTR, BM, BN, WM, WN, true>), grid, block, 0, stream, A, lda, W, ldw, a_scale,
                           w_scale, Y, ldy, acc_out, ld_acc, M, N, K, tiles_m, tiles_n, group_m);
    else
        hipLaunchKernelGGL((w8a8_kernel<INSTR, BM, BN, WM, WN, false>), grid, block, 0, stream, A, lda, W, ldw, a_scale,
                           w_scale, Y, ldy, acc_out, ld_acc, M, N, K, tiles_m, tiles_n, group_m);
    return hipGetLastError();
}

}  // namespace w8a8_impl

using namespace w8a8_impl;

#define BG_W8A8_TILES(X)                       \
    X(BG_MFMA_I32_32X32X32_I8, 128, 128, 2, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 256, 128, 2, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 64, 64, 2, 2)   \
    X(BG_MFMA_I32_16X16X64_I8, 128, 128, 2, 2) \
    X(BG_MFMA_I32_16X16X64_I8, 64, 64, 2, 2)

bool w8a8_has_tile(int mfma, int bm, int bn, int waves_m, int waves_n)
{
#define BG_HAS(I, BM_, BN_, WM_, WN_) \
    if (mfma == I && bm == BM_ && bn == BN_ && waves_m == WM_ && waves_n == WN_) return true;
    BG_W8A8_TILES(BG_HAS)
#undef BG_HAS
    return false;
}

hipError_t launch_w8a8(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y,
                       int64_t ldy, int32_t* acc_out, int64_t ld_acc, hipStream_t stream)
{
#define BG_LAUNCH(I, BM_, BN_, WM_, WN_)                                                                          \
    if (p.mfma == I && p.bm == BM_ && p.bn == BN_ && p.waves_m == WM_ && p.waves_n == WN_)                          \
        return launch<I, BM_, BN_, WM_, WN_>(p, M, N, K, A, lda, W, ldw, a_scale, w_scale, Y, ldy, acc_out, ld_acc, \
                                             stream);
    BG_W8A8_TILES(BG_LAUNCH)
#undef BG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace bg
