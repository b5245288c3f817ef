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
// Two data paths: the pipelined kernel (the default for the 32x32x32
// instruction; see w8a8_pipe_kernel) and a double-buffered one: 128-byte k
// tiles (128 int8) of A and W copied global -> LDS with global_load_lds_dwordx4
// under a row-XOR swizzle; v_mfma_i32_32x32x32_i8 or v_mfma_i32_16x16x64_i8
// with one 16-byte chunk per lane per instruction.
#include <type_traits>

#include "bg_internal.h"
#include "bg_pipe.h"

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

// The pipelined W8A8 kernel: the bf16 pipelined kernel's schedule (a ring
// of NS stages of k tiles copied straight to LDS, one barrier per turn
// placed before the last k-step with the next copies spread among that
// step's MFMAs; or two stages with the next tile's copies in one burst;
// MFMA operands swapped so that a lane holds 4 consecutive columns of one
// row) on v_mfma_i32_32x32x32_i8, whose int32 sum is exact in any order.
// Two or three stages take 128-byte k tiles (every copy fetches whole
// 128-byte lines; three stages of the 128x192 tile hold 120 KB), rings of
// four or more 64-byte ones.  The epilogue applies the fixed order above to
// 4 columns at a time and stages the bf16 tile in LDS for row-contiguous
// 16-byte streaming stores.  A short last k tile (K not a multiple of the
// tile) is copied through registers with zeros past K.
// MODE 0: Y; 1: Y and the int32 accumulators; 2: the accumulators only (no
// scales, no Y: the integer products other paths build on); 3: Y with the
// epilogue's order left free (the bench's free-order twin); 4 and 5: the
// Ozaki-scheme recombination of slice products into fp32 (4) or bf16 (5)
// outputs written through Y (see the epilogue)
template <int BM, int BN, int WM, int WN, int NS, int MODE>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(
    PipeOcc<BM, BN, WM, WN, NS, 1, NS <= 3 ? 128 : 64>::WAVES_PER_EU,
    PipeOcc<BM, BN, WM, WN, NS, 1, NS <= 3 ? 128 : 64>::WAVES_PER_EU)))
void w8a8_pipe_kernel(const int8_t* __restrict__ A, int64_t lda, const int8_t* __restrict__ W, int64_t ldw,
                      const float* __restrict__ a_scale, const float* __restrict__ w_scale,
                      uint16_t* __restrict__ Y, int64_t ldy, int32_t* __restrict__ acc_out, int64_t ld_acc,
                      int64_t M, int64_t N, int64_t K, int tiles_m, int tiles_n, int group_m,
                      const int* __restrict__ ea, const int* __restrict__ eb)
{
    // k tile (bytes), chunks per row, k-steps: 128-byte tiles (whole
    // 128-byte lines per copy) in two stages or a ring of three, 64-byte
    // tiles in a ring of four or more
    constexpr int PK = NS <= 3 ? 128 : 64, PCPR = PK / kChunk, KS = PK / 32;
    constexpr int NW = WM * WN, NT = 64 * NW;
    constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    constexpr int A_CH = BM * PCPR, B_CH = BN * PCPR;
    constexpr int STAGE = A_CH + B_CH;
    constexpr int SLOTS = STAGE / 64, ROUNDS = (SLOTS + NW - 1) / NW, EXTRA = SLOTS % NW;
    constexpr int LOADS_HI = ROUNDS, LOADS_LO = EXTRA ? ROUNDS - 1 : ROUNDS;
    constexpr int CHR = BN / 8;
    constexpr int LDS_BYTES = PipeLds<BM, BN, NS, 1, PK>::BYTES;
    static_assert(A_CH % 64 == 0 && B_CH % 64 == 0, "tile rows must fill whole copy slots");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole MFMA blocks");
    static_assert(NS == 2 || (NS >= 3 && LOADS_HI * (NS - 2) < 64), "stages: three at least, waits within vmcnt");
    static_assert(KS % 2 == 0, "whole pairs of k-steps per turn");
    static_assert(NS != 2 || (EXTRA == 0 && ROUNDS < 64), "128-byte tiles: equal copy rounds");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS holds 160 KiB");
    __shared__ u32x4 lds[LDS_BYTES / 16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int n_full = (int)(K / PK);
    const int n_turns = (int)((K + PK - 1) / PK);
    const bool hi = EXTRA == 0 || wave < EXTRA;

    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) u32x4*)lds);
    // position of logical 16-byte chunk kc in the LDS row `row`: rows of 64
    // bytes swizzled by (row >> 2) & 3, rows of 128 bytes by (row >> 1) & 7
    // (the operand reads of 16 consecutive rows hit 16 distinct bank groups)
    auto kswz = [](int kc, int row) { return PCPR == 4 ? kc ^ ((row >> 2) & 3) : kc ^ ((row >> 1) & 7); };
    const int r_in = lane & 31, h = lane >> 5;
    int a_off[KS], b_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        a_off[ks] = (wm * WTM + r_in) * PCPR + kswz(2 * ks + h, r_in);
        b_off[ks] = A_CH + (wn * WTN + r_in) * PCPR + kswz(2 * ks + h, r_in);
    }
    auto rd = [&](int turn, int ks, i32x4* a, i32x4* b) {
        const u32x4* base = lds + (turn % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < TM; i++) a[i] = __builtin_bit_cast(i32x4, base[a_off[ks] + i * 32 * PCPR]);
#pragma unroll
        for (int j = 0; j < TN; j++) b[j] = __builtin_bit_cast(i32x4, base[b_off[ks] + j * 32 * PCPR]);
    };
    i32x16 acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[j][i][e] = 0;
    auto mm = [&](const i32x4* a, const i32x4* b) {
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++)
                acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j], a[i], acc[j][i], 0, 0, 0);
    };
    if constexpr (NS >= 3) {
        const int8_t* rows[ROUNDS];
        int kcs[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; r++) {
            const int s = r * NW + wave;
            const int c = (s < SLOTS ? s : 0) * 64 + lane;
            const bool is_a = c < A_CH;
            const int row = is_a ? c / PCPR : (c - A_CH) / PCPR;
            kcs[r] = kswz(c % PCPR, row);
            int64_t g = (is_a ? m0 : n0) + row;
            const int64_t lim = is_a ? M : N;
            g = g < lim ? g : lim - 1;  // rows past M or N read a clamped row: never stored
            rows[r] = is_a ? A + g * lda : W + g * ldw;
        }

        // round r of this wave's copies of a whole k tile `turn` (the last
        // round's slots past the stage's end belong to no wave)
        auto copy_round = [&](int turn, int r) {
            const int s = r * NW + wave;
            if (r + 1 < ROUNDS || EXTRA == 0 || s < SLOTS)
                dma16(rows[r] + (int64_t)turn * PK + kcs[r] * kChunk,
                      lds_base + (uint32_t)((turn % NS) * STAGE + s * 64) * 16u);
        };
        auto issue = [&](int turn) {
            const int st = turn % NS;
            const int64_t kb = (int64_t)turn * PK;
#pragma unroll
            for (int r = 0; r < ROUNDS; r++) {
                const int s = r * NW + wave;
                if (r + 1 < ROUNDS || EXTRA == 0 || s < SLOTS) {
                    if (turn < n_full)
                        copy_round(turn, r);
                    else
                        lds[st * STAGE + s * 64 + lane] = load_chunk_i8(rows[r], kb + kcs[r] * kChunk, K);
                }
            }
        };
        auto dma_newer = [&](int after, int last) {
            const int l = last < n_full - 1 ? last : n_full - 1;
            return l > after ? l - after : 0;
        };
        auto wait_newer = [&](int newer, auto max_tag) {
            constexpr int MAXN = decltype(max_tag)::value;
            if (hi) wait_turns<LOADS_HI, MAXN>(newer);
            else wait_turns<LOADS_LO, MAXN>(newer);
        };

        // the same products with this wave's copies of a whole k tile `turn`
        // spread evenly among them (after instruction q of TM TN, the first
        // ROUNDS q / (TM TN) rounds are out) instead of issued in one burst
        auto mm_issue = [&](const i32x4* a, const i32x4* b, int turn) {
            int q = 0, r = 0;
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[j], a[i], acc[j][i], 0, 0, 0);
                    ++q;
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < ROUNDS; u++)
                        if (r < ROUNDS && r * (TM * TN) < ROUNDS * q - (TM * TN - 1)) copy_round(turn, r++);
                    __builtin_amdgcn_sched_barrier(0);
                }
        };

#pragma unroll
        for (int s = 0; s < NS - 1; s++)
            if (s < n_turns) issue(s);
        wait_newer(dma_newer(0, NS - 2), std::integral_constant<int, NS - 2>{});
        __syncthreads();

        i32x4 xa[2][TM], xb[2][TN];
        rd(0, 0, xa[0], xb[0]);
        // k-steps 0 .. KS-2: read the operands of the next k-step, multiply
        // this one (the fragment buffers alternate; KS is even, so the last
        // k-step's operands sit in buffer 1)
        auto turn = [&](int t, auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ks++) {
                rd(t, ks + 1, xa[(ks + 1) & 1], xb[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mm(xa[ks & 1], xb[ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (FULL) {
                if (hi) wait_vmcnt<LOADS_HI * (NS - 3)>();
                else wait_vmcnt<LOADS_LO * (NS - 3)>();
            } else {
                const int last = t + NS - 2 < n_turns - 1 ? t + NS - 2 : n_turns - 1;
                wait_newer(dma_newer(t + 1, last), std::integral_constant<int, NS - 3>{});
            }
            __builtin_amdgcn_s_barrier();
            if constexpr (FULL) {
                rd(t + 1, 0, xa[0], xb[0]);
                __builtin_amdgcn_sched_barrier(0);
                mm_issue(xa[1], xb[1], t + NS - 1);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                if (t + NS - 1 < n_turns) issue(t + NS - 1);
                rd(t + 1, 0, xa[0], xb[0]);  // past the last tile: a stale read, never used
                __builtin_amdgcn_sched_barrier(0);
                mm(xa[1], xb[1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int n_steady = n_full - (NS - 1);
        int t = 0;
        for (; t < n_steady; t++) turn(t, std::true_type{});
        for (; t < n_turns; t++) turn(t, std::false_type{});

    } else {
        // 128-byte k tiles in two stages (as the large bf16 tiles): each
        // lane's copies are addressed from the tile's first row of A or W (a
        // scalar base that walks k) by a fixed 32-bit offset (row within the
        // tile, clamped, times the leading dimension, plus the swizzled
        // chunk); the copies of tile t+1 go out in one burst at the top of
        // turn t, and every wave waits for its copies and its LDS reads of
        // tile t before the turn's barrier.
        const int8_t* const a_base = A + m0 * lda;
        const int8_t* const w_base = W + n0 * ldw;
        uint32_t off[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; r++) {
            const int c = (r * NW + wave) * 64 + lane;
            const bool is_a = c < A_CH;
            const int row = is_a ? c / PCPR : (c - A_CH) / PCPR;
            const int64_t first = is_a ? m0 : n0, lim = is_a ? M : N;
            const int64_t g = first + row < lim ? first + row : lim - 1;
            off[r] = (uint32_t)((g - first) * (is_a ? lda : ldw) + kswz(c % PCPR, row) * kChunk);
        }
        auto slot_base = [&](int s) { return s * 64 < A_CH ? a_base : w_base; };
        auto issue_full = [&](int turn) {
#pragma unroll
            for (int r = 0; r < ROUNDS; r++) {
                const int s = r * NW + wave;
                dma16_off(slot_base(s) + (int64_t)turn * PK, off[r],
                          lds_base + (uint32_t)((turn % NS) * STAGE + s * 64) * 16u);
            }
        };
        // the short last tile (K not a multiple of 128) through registers,
        // zeros past K
        auto issue_short = [&](int turn) {
#pragma unroll
            for (int r = 0; r < ROUNDS; r++) {
                const int s = r * NW + wave;
                const int c = s * 64 + lane;
                const int row = c < A_CH ? c / PCPR : (c - A_CH) / PCPR;
                const int kc = kswz(c % PCPR, row);
                lds[(turn % NS) * STAGE + s * 64 + lane] =
                    load_chunk_i8(slot_base(s) + off[r] - kc * kChunk, (int64_t)turn * PK + kc * kChunk, K);
            }
        };
        if (n_full > 0) issue_full(0);
        else if (n_turns > 0) issue_short(0);
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __syncthreads();
        i32x4 xa[2][TM], xb[2][TN];
        rd(0, 0, xa[0], xb[0]);
        // NEXT: 0 tile t is the last, 1 tile t+1 is whole, 2 it is the short
        // last one
        auto turn = [&](int t, auto next_tag) {
            constexpr int NEXT = decltype(next_tag)::value;
            if constexpr (NEXT == 1) issue_full(t + 1);
            if constexpr (NEXT == 2) issue_short(t + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ks++) {
                rd(t, ks + 1, xa[(ks + 1) & 1], xb[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mm(xa[ks & 1], xb[ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (NEXT != 0) {
                wait_vmcnt<0>();
                wait_lgkmcnt0();
                __builtin_amdgcn_s_barrier();
                rd(t + 1, 0, xa[0], xb[0]);
                __builtin_amdgcn_sched_barrier(0);
            }
            mm(xa[(KS - 1) & 1], xb[(KS - 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
        };
        int t = 0;
        for (; t + 1 < n_full; t++) turn(t, std::integral_constant<int, 1>{});
        if (t + 1 < n_turns) turn(t++, std::integral_constant<int, 2>{});
        if (t < n_turns) turn(t, std::integral_constant<int, 0>{});
    }

    // epilogue: block (j, i), element 4q+u of lane l is row m = wm*WTM + 32i +
    // l%32, column n = wn*WTN + 32j + 8q + 4(l/32) + u
    if constexpr (MODE >= 4) {
        // Ozaki-scheme recombination ("GPU Mechanism", the exact-GEMM
        // paragraph).  The operands are stacked slices, interleaved: stacked
        // row 4m + s is slice s of row m of A, stacked column 4n + t slice t of
        // row n of B, so one 32x32 block of stacked outputs holds all sixteen
        // slice products of 8 x 8 outputs.  Each wave stages its block in LDS
        // as [m'][s][n'][t]; lane (m' = l/8, n' = l%8) reads its sixteen
        // products and sums them in fp64 in the fixed order -- s + t = 6, 5,
        // ..., 0, s ascending within a level, product st weighted 2^-7(s+t+2)
        // -- scales by 2^(ea[m] + eb[n]) and rounds once.
        static_assert(NW * 1024 * 4 <= LDS_BYTES, "a staged block per wave fits in LDS");
        __syncthreads();  // every wave is done with the operand stages
        int32_t* sb = (int32_t*)lds + wave * 1024;
        const int mo = lane >> 3, no = lane & 7;
        const int64_t M4 = M / 4, N4 = N / 4;  // outputs: the stacked sizes are 4 M and 4 N
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++) {
                // lane (r_in = 4 m' + s, h) holds n' = 2q + h, t = 0..3 for q = 0..3
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const i32x4 v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
                    *(i32x4*)(sb + (((r_in >> 2) * 4 + (r_in & 3)) * 8 + 2 * q + h) * 4) = v;
                }
                i32x4 g[4];
#pragma unroll
                for (int s4 = 0; s4 < 4; s4++) g[s4] = *(const i32x4*)(sb + ((mo * 4 + s4) * 8 + no) * 4);
                const int64_t m = (m0 + wm * WTM + 32 * i) / 4 + mo;
                const int64_t n = (n0 + wn * WTN + 32 * j) / 4 + no;
                if (m < M4 && n < N4) {
                    double v = 0.0;
#pragma unroll
                    for (int lev = 6; lev >= 0; lev--)
#pragma unroll
                        for (int s4 = 0; s4 < 4; s4++) {
                            const int t4 = lev - s4;
                            if (t4 < 0 || t4 > 3) continue;
                            v = v + ldexp((double)g[s4][t4], -7 * (lev + 2));
                        }
                    v = ldexp(v, ea[m] + eb[n]);
                    if constexpr (MODE == 5) Y[m * ldy + n] = bf16_from_f64(v);
                    else ((float*)Y)[m * ldy + n] = (float)v;  // one rounding, nearest even
                }
                // the next block's stores follow these loads in this wave's
                // LDS order: no barrier
            }
        return;
    }
    // MODE 3 (free-order twin, bench only): Y with the epilogue's order left
    // free -- one combined scale a_scale * w_scale multiplied in once
    constexpr bool WANT_Y = MODE != 2, WANT_ACC = MODE == 1 || MODE == 2;
    __syncthreads();  // every wave is done with the operand stages
    unsigned char* cl = (unsigned char*)lds;
#pragma unroll
    for (int i = 0; i < TM; i++) {
        const int m = wm * WTM + i * 32 + r_in;
        const int64_t gm = m0 + m;
        float as = 0.0f;
        if constexpr (WANT_Y) as = a_scale[gm < M ? gm : M - 1];
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int n = wn * WTN + j * 32 + 8 * q;  // chunk n/8; lane half h takes bytes 8h..8h+7
                const int64_t gn = n0 + n + 4 * h;
                if constexpr (WANT_Y) {
                    float y[4];
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const float ws = w_scale[gn + u < N ? gn + u : N - 1];
                        const float f = (float)acc[j][i][4 * q + u];  // v_cvt_f32_i32: round to nearest even
                        if constexpr (MODE == 3) {
                            y[u] = f * (as * ws);
                        } else {
                            const float tt = f * ws;  // exact: a power of two
                            y[u] = tt * as;           // the one rounding
                        }
                    }
                    uint2 w;
                    w.x = bf16x2_rne(y[0], y[1]);
                    w.y = bf16x2_rne(y[2], y[3]);
                    *(uint2*)(cl + m * (BN * 2) + c_swizzle<CHR>(n / 8, m) * 16 + h * 8) = w;
                }
                if constexpr (WANT_ACC) {
                    if (gm < M && gn < N) {
                        int32_t* pa = acc_out + gm * ld_acc + gn;
                        if (gn + 4 <= N) {
                            i32x4 v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
                            *(i32x4*)pa = v;
                        } else {
                            for (int u = 0; u < 4 && gn + u < N; u++) pa[u] = acc[j][i][4 * q + u];
                        }
                    }
                }
            }
    }
    if constexpr (WANT_Y) {
        __syncthreads();
        for (int c = tid; c < BM * CHR; c += NT) {
            const int row = c / CHR, ch = c % CHR;
            const int64_t gm = m0 + row, gn = n0 + ch * 8;
            if (gm >= M || gn >= N) continue;
            const u32x4 v = *(const u32x4*)(cl + row * (BN * 2) + c_swizzle<CHR>(ch, row) * 16);
            if (gn + 8 <= N) {
                // streaming store: Y is not read again by this kernel (5 % faster
                // at 1024 x 6144 x 2048)
                __builtin_nontemporal_store(v, (u32x4*)(Y + gm * ldy + gn));
            } else {
                for (int u = 0; u < 8 && gn + u < N; u++) Y[gm * ldy + gn + u] = (uint16_t)(v[u / 2] >> (16 * (u % 2)));
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int NS>
hipError_t launch_pipe(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y,
                       int64_t ldy, int32_t* acc_out, int64_t ld_acc, hipStream_t stream)
{
    if (NS == 2 && !i8_offsets_fit(BM, BN, lda, ldw)) return hipErrorInvalidValue;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int group_m = p.group_m > 0 ? p.group_m : tiles_m;
    dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
    if (p.free_epilogue)  // free-order twin (bench only)
        hipLaunchKernelGGL((w8a8_pipe_kernel<BM, BN, WM, WN, NS, 3>), grid, block, 0, stream, A, lda, W, ldw,
                           a_scale, w_scale, Y, ldy, acc_out, ld_acc, M, N, K, tiles_m, tiles_n, group_m, nullptr,
                           nullptr);
    else if (!Y)
        hipLaunchKernelGGL((w8a8_pipe_kernel<BM, BN, WM, WN, NS, 2>), grid, block, 0, stream, A, lda, W, ldw,
                           a_scale, w_scale, Y, ldy, acc_out, ld_acc, M, N, K, tiles_m, tiles_n, group_m, nullptr,
                           nullptr);
    else if (acc_out)
        hipLaunchKernelGGL((w8a8_pipe_kernel<BM, BN, WM, WN, NS, 1>), grid, block, 0, stream, A, lda, W, ldw,
                           a_scale, w_scale, Y, ldy, acc_out, ld_acc, M, N, K, tiles_m, tiles_n, group_m, nullptr,
                           nullptr);
    else
        hipLaunchKernelGGL((w8a8_pipe_kernel<BM, BN, WM, WN, NS, 0>), grid, block, 0, stream, A, lda, W, ldw,
                           a_scale, w_scale, Y, ldy, acc_out, ld_acc, M, N, K, tiles_m, tiles_n, group_m, nullptr,
                           nullptr);
    return hipGetLastError();
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

// (instruction, BM, BN, waves_m, waves_n, load path: 1 direct-to-LDS double
// buffer, 2 pipelined, LDS stages of the pipelined path)
#define BG_W8A8_TILES(X)                             \
    X(BG_MFMA_I32_32X32X32_I8, 128, 192, 4, 2, 2, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 192, 4, 2, 2, 3) \
    X(BG_MFMA_I32_32X32X32_I8, 256, 256, 2, 4, 2, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 128, 2, 2, 2, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 128, 2, 2, 2, 4) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 128, 2, 2, 2, 5) \
    X(BG_MFMA_I32_32X32X32_I8, 256, 256, 2, 4, 2, 4) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 192, 2, 2, 2, 4) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 192, 2, 2, 2, 5) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 192, 2, 2, 2, 6) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 192, 4, 2, 2, 5) \
    X(BG_MFMA_I32_32X32X32_I8, 128, 64, 2, 2, 2, 8)  \
    X(BG_MFMA_I32_32X32X32_I8, 64, 64, 2, 2, 2, 8)   \
    X(BG_MFMA_I32_32X32X32_I8, 128, 128, 2, 2, 1, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 256, 128, 2, 2, 1, 2) \
    X(BG_MFMA_I32_32X32X32_I8, 64, 64, 2, 2, 1, 2)   \
    X(BG_MFMA_I32_16X16X64_I8, 128, 128, 2, 2, 1, 2) \
    X(BG_MFMA_I32_16X16X64_I8, 64, 64, 2, 2, 1, 2)

// stages == 0 takes the first compiled entry of the shape and path
bool w8a8_has_tile(int mfma, int bm, int bn, int waves_m, int waves_n, int path, int stages)
{
#define BG_HAS(I, BM_, BN_, WM_, WN_, P_, NS_)                                                                  \
    if (mfma == I && bm == BM_ && bn == BN_ && waves_m == WM_ && waves_n == WN_ && path == P_ &&                  \
        (stages == 0 || stages == NS_))                                                                          \
        return true;
    BG_W8A8_TILES(BG_HAS)
#undef BG_HAS
    return false;
}

// one launcher per load path (a kernel launched only from a discarded branch
// would not get its host stub)
template <int P>
struct W8A8Launcher;
template <>
struct W8A8Launcher<1> {
    template <int I, int BM, int BN, int WM, int WN, int NS>
    static hipError_t run(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                          const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y,
                          int64_t ldy, int32_t* acc_out, int64_t ld_acc, hipStream_t stream)
    {
        return launch<I, BM, BN, WM, WN>(p, M, N, K, A, lda, W, ldw, a_scale, w_scale, Y, ldy, acc_out, ld_acc,
                                         stream);
    }
};
template <>
struct W8A8Launcher<2> {
    template <int I, int BM, int BN, int WM, int WN, int NS>
    static hipError_t run(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                          const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y,
                          int64_t ldy, int32_t* acc_out, int64_t ld_acc, hipStream_t stream)
    {
        static_assert(I == BG_MFMA_I32_32X32X32_I8, "the pipelined path runs the 32x32x32 instruction");
        return launch_pipe<BM, BN, WM, WN, NS>(p, M, N, K, A, lda, W, ldw, a_scale, w_scale, Y, ldy, acc_out,
                                               ld_acc, stream);
    }
};

// The pipelined tiles built with the Ozaki recombination epilogue (the ones
// the library picks for the stacked product): BM, BN, waves_m, waves_n, stages.
#define BG_OZAKI_TILES(X) \
    X(256, 256, 2, 4, 2)  \
    X(128, 192, 4, 2, 2)  \
    X(128, 128, 2, 2, 2)  \
    X(64, 64, 2, 2, 8)

template <int BM, int BN, int WM, int WN, int NS>
hipError_t launch_pipe_ozaki(const W8A8Plan& p, int64_t M4, int64_t N4, int64_t Kp, const int8_t* qa,
                             const int8_t* qb, const int* ea, const int* eb, bool out_bf16, void* C, int64_t ldc,
                             hipStream_t stream)
{
    if (NS == 2 && !i8_offsets_fit(BM, BN, Kp, Kp)) return hipErrorInvalidValue;
    const int tiles_m = (int)((M4 + BM - 1) / BM), tiles_n = (int)((N4 + BN - 1) / BN);
    const int group_m = p.group_m > 0 ? p.group_m : tiles_m;
    dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
    if (out_bf16)
        hipLaunchKernelGGL((w8a8_pipe_kernel<BM, BN, WM, WN, NS, 5>), grid, block, 0, stream, qa, Kp, qb, Kp, nullptr,
                           nullptr, (uint16_t*)C, ldc, nullptr, 0, M4, N4, Kp, tiles_m, tiles_n, group_m, ea, eb);
    else
        hipLaunchKernelGGL((w8a8_pipe_kernel<BM, BN, WM, WN, NS, 4>), grid, block, 0, stream, qa, Kp, qb, Kp, nullptr,
                           nullptr, (uint16_t*)C, ldc, nullptr, 0, M4, N4, Kp, tiles_m, tiles_n, group_m, ea, eb);
    return hipGetLastError();
}

bool w8a8_ozaki_has_tile(const W8A8Plan& p)
{
#define BG_OHAS(BM_, BN_, WM_, WN_, NS_)                                                                     \
    if (p.path == 2 && p.mfma == BG_MFMA_I32_32X32X32_I8 && p.bm == BM_ && p.bn == BN_ && p.waves_m == WM_ &&  \
        p.waves_n == WN_ && (p.stages == 0 || p.stages == NS_))                                                \
        return true;
    BG_OZAKI_TILES(BG_OHAS)
#undef BG_OHAS
    return false;
}

hipError_t launch_w8a8_ozaki(const W8A8Plan& p, int64_t M4, int64_t N4, int64_t Kp, const int8_t* qa,
                             const int8_t* qb, const int* ea, const int* eb, bool out_bf16, void* C, int64_t ldc,
                             hipStream_t stream)
{
#define BG_OLAUNCH(BM_, BN_, WM_, WN_, NS_)                                                                  \
    if (p.path == 2 && p.mfma == BG_MFMA_I32_32X32X32_I8 && p.bm == BM_ && p.bn == BN_ && p.waves_m == WM_ &&  \
        p.waves_n == WN_ && (p.stages == 0 || p.stages == NS_))                                                \
        return launch_pipe_ozaki<BM_, BN_, WM_, WN_, NS_>(p, M4, N4, Kp, qa, qb, ea, eb, out_bf16, C, ldc, stream);
    BG_OZAKI_TILES(BG_OLAUNCH)
#undef BG_OLAUNCH
    return hipErrorInvalidValue;
}

hipError_t launch_w8a8(const W8A8Plan& p, int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                       const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale, uint16_t* Y,
                       int64_t ldy, int32_t* acc_out, int64_t ld_acc, hipStream_t stream)
{
    if (!Y && p.path != 2) return hipErrorInvalidValue;  // accumulators only: the pipelined kernel
#define BG_LAUNCH(I, BM_, BN_, WM_, WN_, P_, NS_)                                                              \
    if (p.mfma == I && p.bm == BM_ && p.bn == BN_ && p.waves_m == WM_ && p.waves_n == WN_ && p.path == P_ &&   \
        (p.stages == 0 || p.stages == NS_))                                                                    \
        return W8A8Launcher<P_>::template run<I, BM_, BN_, WM_, WN_, NS_>(p, M, N, K, A, lda, W, ldw, a_scale, \
                                                                         w_scale, Y, ldy, acc_out, ld_acc,     \
                                                                         stream);
    BG_W8A8_TILES(BG_LAUNCH)
#undef BG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace bg
