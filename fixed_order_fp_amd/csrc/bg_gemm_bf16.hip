// bg_gemm_bf16.hip -- order-fixed bf16 GEMM C = A * B^T for gfx950, and the
// fixed-order split-K combine.
//
// Order ("Taming Bitwise Behavior", 3.2.1-3.2.2): every output element owns
// one fp32 accumulator per split, started at +0; the split's k range is walked
// in blocks of instruction_k in ascending k, one MFMA per block, the short last
// block zero-padded.  The tile sizes and the wave grid decide only which lane
// owns which element and how many blocks one LDS turn holds, never which
// products meet in one instruction or in which order the instructions reach
// an accumulator -- so they are free speed knobs.  Split partials are written
// in fp32 and summed by a second kernel, a balanced tree over the split index
// (neighbours first, an odd one carried up), with no atomics; the cast to the
// output type happens once, after the combine.
//
// Data path: A [BM][BK] and B [BN][BK] tiles move global -> registers -> LDS
// (16 B per lane, coalesced along K, 16-B chunks XOR-swizzled by row so that
// the MFMA operand reads, 16 B per lane down 32 rows, hit distinct banks),
// double-buffered with one barrier per turn; MFMA operands are read from LDS
// in the placement of the instruction (lane half h holds k 8h..8h+7).
#include <type_traits>

#include "bg_internal.h"
#include "bg_pipe.h"

namespace bg {

namespace gemm_impl {

constexpr int kChunk = 8;  // bf16 per 16-byte chunk

template <int INSTR>
struct MfmaShape;
template <>
struct MfmaShape<BG_MFMA_F32_32X32X16_BF16> {
    static constexpr int M = 32, N = 32, K = 16, ACC = 16;
    typedef f32x16 acc_t;
};
template <>
struct MfmaShape<BG_MFMA_F32_16X16X32_BF16> {
    static constexpr int M = 16, N = 16, K = 32, ACC = 4;
    typedef f32x4 acc_t;
};

template <int INSTR>
__device__ __forceinline__ typename MfmaShape<INSTR>::acc_t mfma(bf16x8 a, bf16x8 b,
                                                                 typename MfmaShape<INSTR>::acc_t c)
{
    if constexpr (INSTR == BG_MFMA_F32_32X32X16_BF16)
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// One 16-byte chunk of a row: 8 bf16 at k .. k+7, zero beyond k_end or when
// the row is out of range.
__device__ __forceinline__ u32x4 load_chunk(const uint16_t* row_ptr, bool row_ok, int64_t k,
                                            int64_t k_end)
{
    u32x4 v = {0u, 0u, 0u, 0u};
    if (!row_ok || k >= k_end) return v;
    if (k + kChunk <= k_end) return *(const u32x4*)(row_ptr + k);
    uint16_t h[8];
#pragma unroll
    for (int j = 0; j < 8; j++) h[j] = (k + j < k_end) ? row_ptr[k + j] : (uint16_t)0;
    v[0] = h[0] | ((uint32_t)h[1] << 16);
    v[1] = h[2] | ((uint32_t)h[3] << 16);
    v[2] = h[4] | ((uint32_t)h[5] << 16);
    v[3] = h[6] | ((uint32_t)h[7] << 16);
    return v;
}

// LDS position (in u32x4 units) of chunk kc of a tile row; chunks of one row
// are permuted by the low bits of the row index.
template <int BK>
__device__ __forceinline__ int lds_slot(int row, int kc)
{
    constexpr int CPR = BK / kChunk;  // chunks per row
    constexpr int MASK = CPR < 8 ? CPR - 1 : 7;
    return row * CPR + (kc ^ (row & MASK));
}

template <int INSTR, int BM, int BN, int BK, int WM, int WN, bool OUT_BF16, int PARTIAL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, float* __restrict__ ws, int64_t M, int64_t N, Cuts cuts)
{
    typedef MfmaShape<INSTR> S;
    constexpr int NT = 64 * WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
    constexpr int TM = WTM / S::M, TN = WTN / S::N;
    constexpr int CPR = BK / kChunk;
    constexpr int A_CHUNKS = BM * CPR, B_CHUNKS = BN * CPR;
    constexpr int A_PER_T = (A_CHUNKS + NT - 1) / NT, B_PER_T = (B_CHUNKS + NT - 1) / NT;
    static_assert(WTM % S::M == 0 && WTN % S::N == 0, "wave tile must hold whole MFMA blocks");
    static_assert(BK % S::K == 0, "k tile must hold whole instructions");

    __shared__ u32x4 lds_a[2][BM * CPR];
    __shared__ u32x4 lds_b[2][BN * CPR];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int split = blockIdx.z;
    const int64_t k_begin = cuts.c[split];
    const int64_t k_end = cuts.c[split + 1];
    const int n_turns = (int)((k_end - k_begin + BK - 1) / BK);

    typename S::acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < S::ACC; e++) acc[i][j][e] = 0.0f;

    u32x4 ra[A_PER_T], rb[B_PER_T];

    auto global_load = [&](int turn) {
        const int64_t kb = k_begin + (int64_t)turn * BK;
#pragma unroll
        for (int i = 0; i < A_PER_T; i++) {
            const int c = tid + i * NT;
            if (A_CHUNKS % NT == 0 || c < A_CHUNKS) {
                const int row = c / CPR, kc = c % CPR;
                const int64_t gm = m0 + row;
                ra[i] = load_chunk(A + gm * lda, gm < M, kb + kc * kChunk, k_end);
            }
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; i++) {
            const int c = tid + i * NT;
            if (B_CHUNKS % NT == 0 || c < B_CHUNKS) {
                const int row = c / CPR, kc = c % CPR;
                const int64_t gn = n0 + row;
                rb[i] = load_chunk(B + gn * ldb, gn < N, kb + kc * kChunk, k_end);
            }
        }
    };
    auto lds_store = [&](int stage) {
#pragma unroll
        for (int i = 0; i < A_PER_T; i++) {
            const int c = tid + i * NT;
            if (A_CHUNKS % NT == 0 || c < A_CHUNKS) lds_a[stage][lds_slot<BK>(c / CPR, c % CPR)] = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; i++) {
            const int c = tid + i * NT;
            if (B_CHUNKS % NT == 0 || c < B_CHUNKS) lds_b[stage][lds_slot<BK>(c / CPR, c % CPR)] = rb[i];
        }
    };
    auto compute = [&](int stage) {
        // lane's operand row within a block and its chunk offset in a k block
        const int r_in = lane % S::M;
        const int kc_in = lane / S::M;  // 0..1 (32x32x16) or 0..3 (16x16x32)
#pragma unroll
        for (int ks = 0; ks < BK / S::K; ks++) {
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int row = wm * WTM + i * S::M + r_in;
                a[i] = __builtin_bit_cast(bf16x8, lds_a[stage][lds_slot<BK>(row, ks * (S::K / kChunk) + kc_in)]);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int row = wn * WTN + j * S::N + r_in;
                b[j] = __builtin_bit_cast(bf16x8, lds_b[stage][lds_slot<BK>(row, ks * (S::K / kChunk) + kc_in)]);
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) acc[i][j] = mfma<INSTR>(a[i], b[j], acc[i][j]);
        }
    };

    if (n_turns > 0) {
        global_load(0);
        lds_store(0);
        __syncthreads();
        for (int t = 0; t < n_turns; t++) {
            if (t + 1 < n_turns) global_load(t + 1);
            compute(t & 1);
            if (t + 1 < n_turns) lds_store((t + 1) & 1);
            __syncthreads();
        }
    }

    // epilogue: partial to the workspace, or the one rounding to the output
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
                    const float v = acc[i][j][e];
                    if constexpr (PARTIAL == 1)
                        ws[((int64_t)split * M + gm) * N + gn] = v;
                    else if constexpr (PARTIAL == 2)  // free-order twin only
                        unsafeAtomicAdd(&((float*)C)[gm * ldc + gn], v);
                    else if constexpr (OUT_BF16)
                        ((uint16_t*)C)[gm * ldc + gn] = bf16_rne(v);
                    else
                        ((float*)C)[gm * ldc + gn] = v;
                }
            }
}

// 16 bytes from global memory into LDS at lds_dst + 16 * lane (the LDS
// address is taken from the wave's first lane).  The explicit address-space
// casts keep the host pass of a templated kernel well-formed.
__device__ __forceinline__ void lds_copy16(const void* src, u32x4* lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

// The same order as gemm_bf16_kernel, with the operand tiles copied from
// global memory straight into LDS (global_load_lds_dwordx4: lane i of a wave
// writes the 16 bytes it loads to LDS base + 16 i), so no VGPRs and no LDS
// store instructions are spent on staging.  A chunk's LDS slot is fixed by the
// lane that loads it; the lane picks the global chunk (row, logical k chunk)
// that belongs in that slot under the row-XOR swizzle.  Rows past M or N read
// a clamped row: those results are never stored.  A turn that would run past
// the split's k_end is staged through registers with zero fill instead, so a
// short last turn is zero-padded exactly as in the register path.
template <int INSTR, int BM, int BN, int WM, int WN, bool OUT_BF16, int PARTIAL>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_direct_kernel(
    const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B, int64_t ldb,
    void* __restrict__ C, int64_t ldc, float* __restrict__ ws, int64_t M, int64_t N, Cuts cuts,
    int tiles_m, int tiles_n, int group_m)
{
    typedef MfmaShape<INSTR> S;
    constexpr int BK = 64, CPR = BK / kChunk;  // 8 chunks of 16 B per tile row
    constexpr int NW = WM * WN, NT = 64 * NW;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int TM = WTM / S::M, TN = WTN / S::N;
    constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
    constexpr int A_PER_T = A_CH / NT, B_PER_T = B_CH / NT;
    static_assert(A_CH % NT == 0 && B_CH % NT == 0, "tile must split evenly over the waves");
    static_assert(WTM % S::M == 0 && WTN % S::N == 0, "wave tile must hold whole MFMA blocks");

    __shared__ u32x4 lds_a[2][A_CH];
    __shared__ u32x4 lds_b[2][B_CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of(blockIdx.x, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    // the last split (which takes the remainder, so it is the deepest) is
    // dispatched first: longest work first balances the CUs (a schedule
    // choice; each split's chain and the combine are unchanged)
    const int split = (int)gridDim.y - 1 - (int)blockIdx.y;
    const int64_t k_begin = cuts.c[split];
    const int64_t k_end = cuts.c[split + 1];
    const int n_full = (int)((k_end - k_begin) / BK);
    const int n_turns = (int)((k_end - k_begin + BK - 1) / BK);

    // per-lane source rows and logical chunks (fixed for the whole k walk)
    const uint16_t* a_src[A_PER_T];
    const uint16_t* b_src[B_PER_T];
    int a_kc[A_PER_T], b_kc[B_PER_T];
#pragma unroll
    for (int i = 0; i < A_PER_T; i++) {
        const int c = i * NT + wave * 64 + lane;  // LDS slot this lane fills
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
        b_src[i] = B + gn * ldb + b_kc[i] * kChunk;
    }

    typename S::acc_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int e = 0; e < S::ACC; e++) acc[i][j][e] = 0.0f;

    auto issue = [&](int turn, int stage) {
        const int64_t kb = k_begin + (int64_t)turn * BK;
        if (turn < n_full) {
#pragma unroll
            for (int i = 0; i < A_PER_T; i++)
                lds_copy16(a_src[i] + kb, &lds_a[stage][i * NT + wave * 64]);
#pragma unroll
            for (int i = 0; i < B_PER_T; i++)
                lds_copy16(b_src[i] + kb, &lds_b[stage][i * NT + wave * 64]);
        } else {  // the short last turn: zero-filled through registers
#pragma unroll
            for (int i = 0; i < A_PER_T; i++) {
                const int c = i * NT + wave * 64 + lane;
                const int64_t gm = m0 + c / CPR;
                lds_a[stage][c] = load_chunk(A + (gm < M ? gm : M - 1) * lda, true, kb + a_kc[i] * kChunk, k_end);
            }
#pragma unroll
            for (int i = 0; i < B_PER_T; i++) {
                const int c = i * NT + wave * 64 + lane;
                const int64_t gn = n0 + c / CPR;
                lds_b[stage][c] = load_chunk(B + (gn < N ? gn : N - 1) * ldb, true, kb + b_kc[i] * kChunk, k_end);
            }
        }
    };
    auto compute = [&](int stage) {
        const int r_in = lane % S::M;
        const int kc_in = lane / S::M;
#pragma unroll
        for (int ks = 0; ks < BK / S::K; ks++) {
            bf16x8 a[TM], b[TN];
#pragma unroll
            for (int i = 0; i < TM; i++) {
                const int row = wm * WTM + i * S::M + r_in;
                a[i] = __builtin_bit_cast(bf16x8, lds_a[stage][lds_slot<BK>(row, ks * (S::K / kChunk) + kc_in)]);
            }
#pragma unroll
            for (int j = 0; j < TN; j++) {
                const int row = wn * WTN + j * S::N + r_in;
                b[j] = __builtin_bit_cast(bf16x8, lds_b[stage][lds_slot<BK>(row, ks * (S::K / kChunk) + kc_in)]);
            }
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int j = 0; j < TN; j++) acc[i][j] = mfma<INSTR>(a[i], b[j], acc[i][j]);
        }
    };

    if (n_turns > 0) issue(0, 0);
    for (int t = 0; t < n_turns; t++) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this lane's copies have landed
        __syncthreads();                      // ... and every lane's; stage (t+1)&1 is free
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
                    const float v = acc[i][j][e];
                    if constexpr (PARTIAL == 1)
                        ws[((int64_t)split * M + gm) * N + gn] = v;
                    else if constexpr (PARTIAL == 2)  // free-order twin only
                        unsafeAtomicAdd(&((float*)C)[gm * ldc + gn], v);
                    else if constexpr (OUT_BF16)
                        ((uint16_t*)C)[gm * ldc + gn] = bf16_rne(v);
                    else
                        ((float*)C)[gm * ldc + gn] = v;
                }
            }
}

// ---- the pipelined kernel for large M x N --------------------------------
//
// The same order as the kernels above; only the schedule differs.
//  * k tiles of 32 (4 chunks of 16 B per row, swizzled by (row >> 2) & 3 so
//    the operand reads of 16 consecutive rows hit 16 distinct bank groups),
//    NS stages in LDS, turn t+NS-1 copied while turn t is multiplied;
//  * one barrier per turn, placed before the turn's last k-step: the MFMAs
//    of the step before it are still queued while waves meet there, and the
//    first operands of the next turn are read right after it; each wave's
//    copies of the turn NS-1 ahead are then spread among that last k-step's
//    MFMAs;
//  * MFMA operands swapped (the B fragment is the instruction's first operand,
//    so the instruction computes the transposed 32x32 block): every product
//    and every k group is the same, and each lane ends up holding 4
//    consecutive columns of one row of C;
//  * bf16 output is staged through LDS and written row by row, 16 bytes per
//    lane with consecutive lanes on consecutive addresses, as streaming
//    stores.
// The copies bypass the compiler (see dma16) and are waited for explicitly.
//
// BK = 64 (the large tiles) changes the copy schedule: k tiles of 64 (8
// chunks per row, 128 contiguous bytes: each copy instruction fetches whole
// 128-byte lines, half as many L2 requests as 64-byte row pieces), two
// stages, and the copies of tile t+1 issued in one burst at the top of turn
// t, before its first MFMA; every wave waits for its copies and for its LDS
// reads of tile t before the turn's barrier, after which tile t+1's first
// operands are read and tile t's last k-step is multiplied.  Measured 10 %
// faster than the 32-deep ring on the large-output tiles (8 waves, two
// rounds of workgroups or more), bit-identical; on the mid-size tiles (4
// waves, one round) the single tile in flight made it 10-90 % slower.
// Those, and the small tiles, take 64-deep k tiles in a ring of four or
// more stages instead (the same ring as the 32-deep one, four k-steps per
// turn): 8-29 % faster on the small-M and split-K products, where each CU
// streams its operands from HBM; a ring of three measured slower.

// OUT: 0 fp32 C, 1 bf16 C, 2 fp32 split partial to the workspace, 3 fp32
// split partial added into C with atomics, 4 fp32 C from two interleaved
// accumulator chains per output (even k-steps into one, odd into the other,
// the two added once after the walk); 3 and 4 are free-order twins only
// RED: 0 none, 1 and 2 fused reductions of the fp32 C tile (column and row
// leaves; S = 1, OUT 0 or 1).
//
// pipe_tile computes one output tile (walk index b) of one split into the
// workgroup's LDS `lds`; the kernels below map workgroups to (b, split).
template <int BM, int BN, int WM, int WN, int NS, int OUT, int RED, int BK = 32>
__device__ __forceinline__ void pipe_tile(u32x4* __restrict__ lds, int b, int split,
                                          const uint16_t* __restrict__ A, int64_t lda,
                                          const uint16_t* __restrict__ B, int64_t ldb, void* __restrict__ C,
                                          int64_t ldc, float* __restrict__ ws, int64_t M, int64_t N,
                                          const Cuts& cuts, int tiles_m, int tiles_n, int group_m,
                                          const RedArgs& red)
{
    constexpr int CPR = BK / kChunk, KS = BK / 16;
    constexpr int NW = WM * WN, NT = 64 * NW;
    constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 32, TN = WTN / 32;
    constexpr int A_CH = BM * CPR, B_CH = BN * CPR;
    constexpr int STAGE = A_CH + B_CH;  // 16-byte chunks per stage
    // a stage is copied in slots of 64 chunks (one instruction per wave); slot
    // s goes to wave s % NW in round s / NW, so waves below SLOTS % NW make
    // one copy more per tile than the others
    constexpr int SLOTS = STAGE / 64, ROUNDS = (SLOTS + NW - 1) / NW, EXTRA = SLOTS % NW;
    constexpr int LOADS_HI = ROUNDS, LOADS_LO = EXTRA ? ROUNDS - 1 : ROUNDS;
    constexpr int CHR = BN / 8;  // 16-byte chunks per staged bf16 C row
    constexpr int LDS_BYTES = PipeLds<BM, BN, NS, OUT, BK * 2>::BYTES;
    static_assert(A_CH % 64 == 0 && B_CH % 64 == 0, "tile rows must fill whole copy slots");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must hold whole MFMA blocks");
    static_assert(BK == 32 || BK == 64, "k tiles of 32 or 64");
    static_assert(OUT != 4 || (RED == 0 && KS % 2 == 0), "two chains: fp32 C, whole pairs of k-steps per turn");
    static_assert(NS == 2 || (NS >= 3 && LOADS_HI * (NS - 2) < 64), "a ring of three stages at least, waits within vmcnt");
    static_assert(NS != 2 || (BK == 64 && EXTRA == 0 && ROUNDS < 64), "two stages: 64-deep tiles, equal copy rounds");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS holds 160 KiB");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int tm, tn;
    tile_of(b, tiles_m, tiles_n, group_m, tm, tn);
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * BN;
    const int64_t k_begin = cuts.c[split];
    const int64_t k_end = cuts.c[split + 1];
    const int n_full = (int)((k_end - k_begin) / BK);
    const int n_turns = (int)((k_end - k_begin + BK - 1) / BK);
    const bool hi = EXTRA == 0 || wave < EXTRA;  // this wave copies ROUNDS slots

    const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) u32x4*)lds);
    // position of logical 16-byte chunk kc in the LDS row `row` (an XOR by a
    // few row bits, so that the operand reads of 16 consecutive rows hit 16
    // distinct bank groups): rows of 64 bytes by (row >> 2) & 3, rows of 128
    // bytes by (row >> 1) & 7
    auto kswz = [](int kc, int row) { return CPR == 4 ? kc ^ ((row >> 2) & 3) : kc ^ ((row >> 1) & 7); };
    // operand fragment offsets (in chunks) for the k-steps of a turn; the
    // 32-row blocks of a wave add multiples of 32 rows, which keep the swizzle
    const int r_in = lane & 31, h = lane >> 5;
    int a_off[KS], b_off[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
        a_off[ks] = (wm * WTM + r_in) * CPR + kswz(2 * ks + h, r_in);
        b_off[ks] = A_CH + (wn * WTN + r_in) * CPR + kswz(2 * ks + h, r_in);
    }
    auto rd = [&](int turn, int ks, bf16x8* a, bf16x8* b) {
        const u32x4* base = lds + (turn % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < TM; i++) a[i] = __builtin_bit_cast(bf16x8, base[a_off[ks] + i * 32 * CPR]);
#pragma unroll
        for (int j = 0; j < TN; j++) b[j] = __builtin_bit_cast(bf16x8, base[b_off[ks] + j * 32 * CPR]);
    };

    f32x16 acc[TN][TM];  // block (j, i): rows n of C^T = columns n of C
    constexpr bool TWO = OUT == 4;
    f32x16 acc2[TWO ? TN : 1][TWO ? TM : 1];  // the odd k-steps' chain (OUT 4)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[j][i][e] = 0.0f;
    if constexpr (TWO) {
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int e = 0; e < 16; e++) acc2[j][i][e] = 0.0f;
    }
    // one instruction into block (j, i); `odd` (the k-step's parity, a
    // constant once the loops are unrolled) picks the chain under OUT 4
    auto mfma1 = [&](int j, int i, const bf16x8& a, const bf16x8& b, int odd) {
        if constexpr (TWO) {
            if (odd) {
                acc2[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc2[j][i], 0, 0, 0);
                return;
            }
        }
        acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, acc[j][i], 0, 0, 0);
    };
    auto mm = [&](const bf16x8* a, const bf16x8* b, int odd) {
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++) mfma1(j, i, a[i], b[j], odd);
    };
    if constexpr (NS >= 3) {
        // the chunk this lane copies in round r: stage chunk c = 64 s + lane (A
        // rows first, then B rows), global (row, logical chunk kc) under the swizzle
        const uint16_t* src[ROUNDS];
        int kcs[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; r++) {
            const int s = r * NW + wave;
            const int c = (s < SLOTS ? s : 0) * 64 + lane;
            const bool is_a = c < A_CH;
            const int row = is_a ? c / CPR : (c - A_CH) / CPR;
            kcs[r] = kswz(c % CPR, row);
            int64_t g = (is_a ? m0 : n0) + row;
            const int64_t lim = is_a ? M : N;
            g = g < lim ? g : lim - 1;  // rows past M or N read a clamped row: never stored
            src[r] = (is_a ? A + g * lda : B + g * ldb) + k_begin + kcs[r] * kChunk;
        }

        // copy k tile `turn` into its stage; the short last tile (k_end not a
        // multiple of 32 past k_begin) goes through registers with zeros past
        // k_end (cut points are multiples of 8, so a chunk is all in or all out)
        // round r of this wave's copies of a whole k tile `turn` (the last
        // round's slots past the stage's end belong to no wave)
        auto copy_round = [&](int turn, int r) {
            const int s = r * NW + wave;
            if (r + 1 < ROUNDS || EXTRA == 0 || s < SLOTS)
                dma16(src[r] + (int64_t)turn * BK, lds_base + (uint32_t)((turn % NS) * STAGE + s * 64) * 16u);
        };
        auto issue = [&](int turn) {
            const int st = turn % NS;
            const int64_t kb = (int64_t)turn * BK;
#pragma unroll
            for (int r = 0; r < ROUNDS; r++) {
                const int s = r * NW + wave;
                if (r + 1 < ROUNDS || EXTRA == 0 || s < SLOTS) {
                    if (turn < n_full) {
                        copy_round(turn, r);
                    } else {
                        u32x4 v = {0u, 0u, 0u, 0u};
                        if (k_begin + kb + kcs[r] * kChunk < k_end) v = *(const u32x4*)(src[r] + kb);
                        lds[st * STAGE + s * 64 + lane] = v;
                    }
                }
            }
        };
        // copied turns after turn `after` that may still be in flight once turns
        // up to `last` have been issued (the short tile is synchronous)
        auto dma_newer = [&](int after, int last) {
            const int l = last < n_full - 1 ? last : n_full - 1;
            return l > after ? l - after : 0;
        };
        // wait until at most `newer` turns of this wave's copies are outstanding
        auto wait_newer = [&](int newer, auto max_tag) {
            constexpr int MAXN = decltype(max_tag)::value;
            if (hi) wait_turns<LOADS_HI, MAXN>(newer);
            else wait_turns<LOADS_LO, MAXN>(newer);
        };

        // the same products with this wave's copies of a whole k tile `turn`
        // spread evenly among them (after instruction q of TM TN, the first
        // ROUNDS q / (TM TN) rounds are out) instead of issued in one burst ahead
        // of them: measured 3-5 % faster on the large tiles
        auto mm_issue = [&](const bf16x8* a, const bf16x8* b, int turn) {
            int q = 0, r = 0;
#pragma unroll
            for (int j = 0; j < TN; j++)
#pragma unroll
                for (int i = 0; i < TM; i++) {
                    mfma1(j, i, a[i], b[j], 1);  // the last k-step of a turn (KS is even)
                    ++q;
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int u = 0; u < ROUNDS; u++)
                        if (r < ROUNDS && r * (TM * TN) < ROUNDS * q - (TM * TN - 1)) copy_round(turn, r++);
                    __builtin_amdgcn_sched_barrier(0);
                }
        };

        // prologue: tiles 0 .. NS-2 in flight, tile 0 landed and visible
#pragma unroll
        for (int s = 0; s < NS - 1; s++)
            if (s < n_turns) issue(s);
        wait_newer(dma_newer(0, NS - 2), std::integral_constant<int, NS - 2>{});
        __syncthreads();

        bf16x8 xa[2][TM], xb[2][TN];
        rd(0, 0, xa[0], xb[0]);
        // FULL: tiles t+1 .. t+NS-1 are all whole, so every wait and copy is
        // unconditional and the loop body has no branch (the compiler can then
        // count LDS reads across the back edge)
        auto turn = [&](int t, auto full_tag) {
            constexpr bool FULL = decltype(full_tag)::value;
            // k-steps 0 .. KS-2: read the operands of the next k-step,
            // multiply this one (the fragment buffers alternate)
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ks++) {
                rd(t, ks + 1, xa[(ks + 1) & 1], xb[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mm(xa[ks & 1], xb[ks & 1], ks & 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            // tile t+1 must have landed in every wave's share before its first read
            if constexpr (FULL) {
                if (hi) wait_vmcnt<LOADS_HI * (NS - 3)>();
                else wait_vmcnt<LOADS_LO * (NS - 3)>();
            } else {
                const int last = t + NS - 2 < n_turns - 1 ? t + NS - 2 : n_turns - 1;
                wait_newer(dma_newer(t + 1, last), std::integral_constant<int, NS - 3>{});
            }
            __builtin_amdgcn_s_barrier();
            // every wave is past its reads of tile t-1: its stage takes tile t+NS-1
            if constexpr (FULL) {
                rd(t + 1, 0, xa[0], xb[0]);
                __builtin_amdgcn_sched_barrier(0);
                mm_issue(xa[1], xb[1], t + NS - 1);
                __builtin_amdgcn_sched_barrier(0);
            } else {
                if (t + NS - 1 < n_turns) issue(t + NS - 1);
                rd(t + 1, 0, xa[0], xb[0]);  // past the last tile: a stale read, never used
                __builtin_amdgcn_sched_barrier(0);
                mm(xa[1], xb[1], 1);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int n_steady = n_full - (NS - 1);
        int t = 0;
        for (; t < n_steady; t++) turn(t, std::true_type{});
        for (; t < n_turns; t++) turn(t, std::false_type{});

    } else {
        // 64-deep k tiles, two stages.  Each lane's copies are addressed from
        // the tile's first row of A or B and the split's first k (a scalar
        // base that walks k) by a fixed 32-bit byte offset: row within the
        // tile (rows past M or N clamped to the last one, never stored) times
        // the leading dimension, plus the swizzled chunk.  The host keeps
        // (tile rows - 1) x leading dimension x 2 bytes below 2^32.
        const uint16_t* const a_base = A + m0 * lda + k_begin;
        const uint16_t* const b_base = B + n0 * ldb + k_begin;
        uint32_t off[ROUNDS];
#pragma unroll
        for (int r = 0; r < ROUNDS; r++) {
            const int c = (r * NW + wave) * 64 + lane;
            const bool is_a = c < A_CH;
            const int row = is_a ? c / CPR : (c - A_CH) / CPR;
            const int64_t first = is_a ? m0 : n0, lim = is_a ? M : N;
            const int64_t g = first + row < lim ? first + row : lim - 1;
            off[r] = (uint32_t)(((g - first) * (is_a ? lda : ldb) + kswz(c % CPR, row) * kChunk) * 2);
        }
        // slot s of a stage holds A rows below A_CH / 64, B rows above
        auto slot_base = [&](int s) { return s * 64 < A_CH ? a_base : b_base; };
        // copy k tile `turn` into stage turn % 2: a whole tile with the direct
        // copies; the short last tile (k_end not a multiple of 64 past
        // k_begin) through registers, zeros past k_end (cut points are
        // multiples of 8, so a chunk is all in or all out)
        auto issue_full = [&](int turn) {
#pragma unroll
            for (int r = 0; r < ROUNDS; r++) {
                const int s = r * NW + wave;
                dma16_off(slot_base(s) + (int64_t)turn * BK, off[r],
                          lds_base + (uint32_t)((turn % NS) * STAGE + s * 64) * 16u);
            }
        };
        auto issue_short = [&](int turn) {
#pragma unroll
            for (int r = 0; r < ROUNDS; r++) {
                const int s = r * NW + wave;
                const int c = s * 64 + lane;
                const int row = c < A_CH ? c / CPR : (c - A_CH) / CPR;
                const int64_t k = (int64_t)turn * BK + kswz(c % CPR, row) * kChunk;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (k_begin + k < k_end)
                    v = *(const u32x4*)((const unsigned char*)(slot_base(s) + (int64_t)turn * BK) + off[r]);
                lds[(turn % NS) * STAGE + s * 64 + lane] = v;
            }
        };
        if (n_full > 0) issue_full(0);
        else if (n_turns > 0) issue_short(0);
        wait_vmcnt<0>();
        wait_lgkmcnt0();
        __syncthreads();
        bf16x8 xa[2][TM], xb[2][TN];
        rd(0, 0, xa[0], xb[0]);
        // NEXT: 0 tile t is the last, 1 tile t+1 is whole, 2 tile t+1 is the
        // short last one.  Tile t+1's copies go out at the top of the turn,
        // into the stage of tile t-1, whose reads every wave finished before
        // the last barrier.
        auto turn = [&](int t, auto next_tag) {
            constexpr int NEXT = decltype(next_tag)::value;
            if constexpr (NEXT == 1) issue_full(t + 1);
            if constexpr (NEXT == 2) issue_short(t + 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ks++) {
                rd(t, ks + 1, xa[(ks + 1) & 1], xb[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                mm(xa[ks & 1], xb[ks & 1], ks & 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            if constexpr (NEXT != 0) {
                // tile t+1 landed in every wave's share, and this wave's reads
                // of tile t have returned: after the barrier tile t's stage is
                // free and tile t+1 is visible
                wait_vmcnt<0>();
                wait_lgkmcnt0();
                __builtin_amdgcn_s_barrier();
                rd(t + 1, 0, xa[0], xb[0]);
                __builtin_amdgcn_sched_barrier(0);
            }
            mm(xa[(KS - 1) & 1], xb[(KS - 1) & 1], (KS - 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
        };
        int t = 0;
        for (; t + 1 < n_full; t++) turn(t, std::integral_constant<int, 1>{});
        if (t + 1 < n_turns) turn(t++, std::integral_constant<int, 2>{});
        if (t < n_turns) turn(t, std::integral_constant<int, 0>{});
    }

    if constexpr (TWO) {  // the two chains, added once per output
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int e = 0; e < 16; e++) acc[j][i][e] = acc[j][i][e] + acc2[j][i][e];
    }

    // Block (j, i), element e of lane l: row m = wm*WTM + 32i + l%32, columns
    // n = wn*WTN + 32j + 8(e/4) + 4(l/32) + (0..3) for e%4 = 0..3.
    //

    // epilogue
    if constexpr (OUT == 1) {
        __syncthreads();  // every wave is done with the operand stages
        unsigned char* cl = (unsigned char*)lds;
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int m = wm * WTM + i * 32 + r_in;
                    const int n = wn * WTN + j * 32 + 8 * q;  // chunk n/8; lane half h takes bytes 8h..8h+7
                    uint2 w;
                    w.x = bf16x2_rne(acc[j][i][4 * q + 0], acc[j][i][4 * q + 1]);
                    w.y = bf16x2_rne(acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]);
                    *(uint2*)(cl + m * (BN * 2) + c_swizzle<CHR>(n / 8, m) * 16 + h * 8) = w;
                }
        __syncthreads();
        uint16_t* Cb = (uint16_t*)C;
        for (int c = tid; c < BM * CHR; c += NT) {
            const int row = c / CHR, ch = c % CHR;
            const int64_t gm = m0 + row, gn = n0 + ch * 8;
            if (gm >= M || gn >= N) continue;
            const u32x4 v = *(const u32x4*)(cl + row * (BN * 2) + c_swizzle<CHR>(ch, row) * 16);
            if (gn + 8 <= N) {
                // streaming store: the C tile is not read again by this kernel
                // (5-6 % faster where C is large against the run, M = 512)
                __builtin_nontemporal_store(v, (u32x4*)(Cb + gm * ldc + gn));
            } else {
                for (int u = 0; u < 8 && gn + u < N; u++)
                    Cb[gm * ldc + gn + u] = (uint16_t)(v[u / 2] >> (16 * (u % 2)));
            }
        }
    } else if constexpr (OUT == 3) {
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const int64_t gm = m0 + wm * WTM + i * 32 + r_in;
                    const int64_t gn = n0 + wn * WTN + j * 32 + 8 * q + 4 * h;
                    if (gm >= M || gn >= N) continue;
                    float* p = (float*)C + gm * ldc + gn;
                    for (int u = 0; u < 4 && gn + u < N; u++) unsafeAtomicAdd(p + u, acc[j][i][4 * q + u]);
                }
    } else {
        // fp32 C or a split's partial plane: each wave stages one 32x32 block
        // at a time in its own LDS slice (rows of 36 floats keep every row
        // 16-byte aligned) and writes it back as 8 rows of 128 contiguous
        // bytes per store instruction, instead of 32 rows of 32 bytes from the
        // MFMA layout.  Only this wave reads its slice: the LDS keeps one
        // wave's accesses in order, so no barrier is needed between blocks.
        constexpr int PITCH = 36;
        static_assert(NW * 32 * PITCH * 4 <= LDS_BYTES, "the store slices fit in LDS");
        float* out = OUT == 2 ? ws + (int64_t)split * M * N : (float*)C;
        const int64_t ld = OUT == 2 ? N : ldc;
        const bool vec_ok = (ld % 4) == 0;
        __syncthreads();  // every wave is done with the operand stages
        float* st = (float*)lds + wave * (32 * PITCH);
        const int rr = lane >> 3, cc = (lane & 7) * 4;  // this lane's row (of 8) and column in a store
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
            for (int i = 0; i < TM; i++) {
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    f32x4 v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2], acc[j][i][4 * q + 3]};
                    *(f32x4*)(st + r_in * PITCH + 8 * q + 4 * h) = v;
                }
                const int64_t gn = n0 + wn * WTN + j * 32 + cc;
#pragma unroll
                for (int pass = 0; pass < 4; pass++) {
                    const int row = 8 * pass + rr;
                    const f32x4 v = *(const f32x4*)(st + row * PITCH + cc);
                    const int64_t gm = m0 + wm * WTM + i * 32 + row;
                    if (gm >= M || gn >= N) continue;
                    float* p = out + gm * ld + gn;
                    if (vec_ok && gn + 4 <= N) {
                        *(f32x4*)p = v;
                    } else {
                        for (int u = 0; u < 4 && gn + u < N; u++) p[u] = v[u];
                    }
                }
            }
    }

    // Fused reductions of the fp32 C values (before any rounding to the output
    // type), after the C epilogue -- the accumulators are still in
    // registers, and the C tile's global stores drain during the fold: each
    // wave stages two 32x32 blocks at a time in its own LDS slice
    // (rows of 36 floats, the second block 32 banks over, so that a column
    // walk is free of bank conflicts and a row walk reads 16 bytes at a time);
    // lane c of each half-wave folds column c of its block over the rows
    // (RED 1: a leaf of 32 rows) or row c over the columns (RED 2: a leaf of
    // 32 columns) in index order, with no seed (s = x0, s = s + xi; q = x0 x0,
    // q = fma(xi, xi, q) or q + xi xi), and writes the leaf node.  The leaf's
    // elements past M or N are left out (a short last leaf).
    if constexpr (RED != 0) {
        static_assert(OUT == 0 || OUT == 1, "fused reductions take the unsplit C");
        constexpr int RP = 36;                     // floats per staged row (16-byte aligned)
        constexpr int BLK = 32 * RP + 32;          // one staged block; the second one 32 banks over
        constexpr int NB = TM * TN;
        static_assert(NW * 2 * BLK * 4 <= LDS_BYTES, "the reduction slices fit in LDS");
        // every wave is done with the C tile's staging in LDS (its reads have
        // returned): the fold reuses the LDS while the C stores drain
        wait_lgkmcnt0();
        __builtin_amdgcn_s_barrier();
        float* st = (float*)lds + wave * (2 * BLK);
        const int half = lane >> 5, c = lane & 31;
        // blocks b = 2p and 2p + 1 are staged together; lanes 0..31 fold
        // the leaves of the first, lanes 32..63 those of the second
        auto fold_all = [&](auto fused_tag) {
            constexpr bool FUSED = decltype(fused_tag)::value;
            auto step = [&](float v, float& sv, float& qv) {
                sv = sv + v;
                if constexpr (FUSED) {
                    qv = __builtin_fmaf(v, v, qv);
                } else {
                    const float vv = v * v;
                    qv = qv + vv;
                }
            };
#pragma unroll
            for (int p = 0; p < (NB + 1) / 2; p++) {
#pragma unroll
                for (int k = 0; k < 2; k++) {
                    if (2 * p + k < NB) {
                        const int j = (2 * p + k) / TM, i = (2 * p + k) % TM;
                        float* sb = st + k * BLK;
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const f32x4 v = {acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                                             acc[j][i][4 * q + 3]};
                            *(f32x4*)(sb + r_in * RP + 8 * q + 4 * h) = v;
                        }
                    }
                }
                const int b = 2 * p + half;
                const int j = b / TM, i = b % TM;
                const int64_t rb = m0 + wm * WTM + 32 * i, cb = n0 + wn * WTN + 32 * j;
                const int64_t n_el = RED == 1 ? M - rb : N - cb;  // elements of this lane's leaf
                const int64_t o = (RED == 1 ? cb : rb) + c;        // this lane's output
                const int64_t o_end = RED == 1 ? N : M;
                if (b < NB && o < o_end && n_el > 0) {
                    const int n = n_el < 32 ? (int)n_el : 32;
                    const float* sb = st + half * BLK;
                    float sv, qv;
                    if (n == 32) {  // a whole leaf: its 32 elements are read at once, then folded
                        float xv[32];
                        if constexpr (RED == 1) {  // column c, down the rows
#pragma unroll
                            for (int e = 0; e < 32; e++) xv[e] = sb[c + RP * e];
                        } else {  // row c, along the columns
#pragma unroll
                            for (int e = 0; e < 32; e += 4) {
                                const f32x4 v = *(const f32x4*)(sb + c * RP + e);
                                xv[e] = v[0], xv[e + 1] = v[1], xv[e + 2] = v[2], xv[e + 3] = v[3];
                            }
                        }
                        sv = xv[0], qv = xv[0] * xv[0];
#pragma unroll
                        for (int e = 1; e < 32; e++) step(xv[e], sv, qv);
                    } else {  // the short last leaf
                        constexpr int STEP = RED == 1 ? RP : 1;
                        const float* x = sb + (RED == 1 ? c : c * RP);
                        sv = x[0], qv = x[0] * x[0];
                        for (int e = 1; e < n; e++) step(x[e * STEP], sv, qv);
                    }
                    const int64_t leaf = (RED == 1 ? rb : cb) / 32;
                    if (red.ws_sum) red.ws_sum[leaf * red.n_out + o] = sv;
                    if (red.ws_sq) red.ws_sq[leaf * red.n_out + o] = qv;
                }
            }
        };
        if (red.fused) fold_all(std::true_type{});
        else fold_all(std::false_type{});
    }
}

// One tile shape for every split: workgroup x walks the tiles, y the splits.
// The last split (which takes the remainder, so it is the deepest) is
// dispatched first: longest work first balances the CUs (a schedule choice;
// each split's chain and the combine are unchanged).
template <int BM, int BN, int WM, int WN, int NS, int OUT, int RED = 0, int BK = 32>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(
    PipeOcc<BM, BN, WM, WN, NS, OUT, BK * 2>::WAVES_PER_EU, PipeOcc<BM, BN, WM, WN, NS, OUT, BK * 2>::WAVES_PER_EU)))
void gemm_bf16_pipe_kernel(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
                           int64_t ldb, void* __restrict__ C, int64_t ldc, float* __restrict__ ws, int64_t M,
                           int64_t N, Cuts cuts, int tiles_m, int tiles_n, int group_m, RedArgs red)
{
    __shared__ u32x4 lds[PipeLds<BM, BN, NS, OUT, BK * 2>::BYTES / 16];
    pipe_tile<BM, BN, WM, WN, NS, OUT, RED, BK>(lds, (int)blockIdx.x, (int)gridDim.y - 1 - (int)blockIdx.y, A, lda,
                                                B, ldb, C, ldc, ws, M, N, cuts, tiles_m, tiles_n, group_m, red);
}

// Two tile shapes in one launch: the last split (the cut rule's remainder,
// the deepest) takes tile BM2 x BN2, the other splits BM x BN.  A deep split
// on the large tile would be the critical path (few workgroups, many k
// tiles), on the small tile of every split the copies would grow with
// 1/BM + 1/BN; both shapes share the launch so that the CUs stay busy
// through both.  The workgroups of the last split come first when
// `last_first` is set, else last.  Both shapes take the same k tile depth
// BK.  Only the schedule differs: every split's chain is the one its k range
// gives, and its partial plane is the same.
template <int BM, int BN, int WM, int WN, int NS, int BM2, int BN2, int WM2, int WN2, int NS2, int BK = 32>
struct DualLds {
    static constexpr int A = PipeLds<BM, BN, NS, 2, BK * 2>::BYTES, B = PipeLds<BM2, BN2, NS2, 2, BK * 2>::BYTES;
    static constexpr int BYTES = A > B ? A : B;
    static constexpr int W0 = (160 * 1024) / BYTES * WM * WN / 4;
    static constexpr int WAVES_PER_EU = W0 < 1 ? 1 : W0;
};

// OUT: 2 partial planes in the workspace, 3 partials added into C with
// atomics (the free-order twin only).
template <int BM, int BN, int WM, int WN, int NS, int BM2, int BN2, int WM2, int WN2, int NS2, int OUT,
          int BK = 32>
__global__ __launch_bounds__(64 * WM * WN) __attribute__((amdgpu_waves_per_eu(
    DualLds<BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, BK>::WAVES_PER_EU,
    DualLds<BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, BK>::WAVES_PER_EU)))
void gemm_bf16_pipe_dual_kernel(const uint16_t* __restrict__ A, int64_t lda, const uint16_t* __restrict__ B,
                                int64_t ldb, void* __restrict__ C, int64_t ldc, float* __restrict__ ws, int64_t M,
                                int64_t N, Cuts cuts, int S, int tiles_m, int tiles_n, int group_m, int tiles_m2,
                                int tiles_n2, int group_m2, int last_first)
{
    static_assert(OUT == 2 || OUT == 3, "split partials only");
    static_assert(WM * WN == WM2 * WN2, "both shapes run with the workgroup's waves");
    __shared__ u32x4 lds[DualLds<BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, BK>::BYTES / 16];
    const int n_last = tiles_m2 * tiles_n2, n_body = tiles_m * tiles_n * (S - 1);
    int b = (int)blockIdx.x;
    bool is_last;
    if (last_first) {
        is_last = b < n_last;
        if (!is_last) b -= n_last;
    } else {
        is_last = b >= n_body;
        if (is_last) b -= n_body;
    }
    if (is_last) {
        pipe_tile<BM2, BN2, WM2, WN2, NS2, OUT, 0, BK>(lds, b, S - 1, A, lda, B, ldb, C, ldc, ws, M, N, cuts, tiles_m2,
                                                   tiles_n2, group_m2, RedArgs{});
    } else {
        const int T = tiles_m * tiles_n;
        pipe_tile<BM, BN, WM, WN, NS, OUT, 0, BK>(lds, b % T, b / T, A, lda, B, ldb, C, ldc, ws, M, N, cuts, tiles_m,
                                              tiles_n, group_m, RedArgs{});
    }
}

// Balanced tree over v[0..n), neighbours first, an odd last element carried
// up unchanged.  With n a compile-time constant the loops unroll and v stays
// in registers.
template <int NS>
__device__ __forceinline__ float tree_fixed(float (&v)[NS])
{
    int n = NS;
#pragma unroll
    for (int level = 0; level < 7; level++) {
        if (n <= 1) break;
        int w = 0;
#pragma unroll
        for (int i = 0; i + 1 < NS; i += 2)
            if (i + 1 < n) v[w++] = v[i] + v[i + 1];
        if (n & 1) v[w++] = v[n - 1];
        n = w;
    }
    return v[0];
}

__device__ __forceinline__ float tree_dyn(float* v, int n)
{
    while (n > 1) {
        int w = 0;
        for (int i = 0; i + 1 < n; i += 2) v[w++] = v[i] + v[i + 1];
        if (n & 1) v[w++] = v[n - 1];
        n = w;
    }
    return v[0];
}

template <int NS, bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_combine_kernel(const float* __restrict__ ws, int S,
                                                             int64_t M, int64_t N, void* __restrict__ C,
                                                             int64_t ldc)
{
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= M * N) return;
    const int64_t m = idx / N, n = idx % N;
    const int64_t plane = M * N;
    float r;
    if constexpr (NS > 0) {
        float v[NS];
#pragma unroll
        for (int s = 0; s < NS; s++) v[s] = ws[s * plane + idx];
        r = tree_fixed<NS>(v);
    } else {
        float v[BG_MAX_SPLIT];
        for (int s = 0; s < S; s++) v[s] = ws[s * plane + idx];
        r = tree_dyn(v, S);
    }
    if constexpr (OUT_BF16)
        ((uint16_t*)C)[m * ldc + n] = bf16_rne(r);
    else
        ((float*)C)[m * ldc + n] = r;
}

// One launcher per staging path (a kernel launched from one branch of an
// `if constexpr` does not get its host stub emitted, so the two paths are two
// specialisations).
template <int DIRECT>
struct TileLauncher;

template <>
struct TileLauncher<1> {
    template <int INSTR, int BM, int BN, int BK, int WM, int WN, int NS>
    static hipError_t run(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb, void* C, int64_t ldc, float* ws, hipStream_t stream)
    {
        static_assert(BK == 64, "the direct path stages k tiles of 64");
        const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
        const int group_m = p.group_m > 0 ? p.group_m : 8;
        dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)p.S), block(64 * WM * WN);
        if (p.atomic)
            hipLaunchKernelGGL((gemm_bf16_direct_kernel<INSTR, BM, BN, WM, WN, false, 2>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m);
        else if (p.S > 1)
            hipLaunchKernelGGL((gemm_bf16_direct_kernel<INSTR, BM, BN, WM, WN, false, 1>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m);
        else if (p.out_bf16)
            hipLaunchKernelGGL((gemm_bf16_direct_kernel<INSTR, BM, BN, WM, WN, true, 0>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m);
        else
            hipLaunchKernelGGL((gemm_bf16_direct_kernel<INSTR, BM, BN, WM, WN, false, 0>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m);
        return hipGetLastError();
    }
};

template <>
struct TileLauncher<2> {
    template <int INSTR, int BM, int BN, int BK, int WM, int WN, int NS>
    static hipError_t run(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb, void* C, int64_t ldc, float* ws, hipStream_t stream)
    {
        static_assert(INSTR == BG_MFMA_F32_32X32X16_BF16 && (BK == 32 || BK == 64),
                      "the pipelined path: 32x32x16, k tiles of 32 or 64");
        if (BK == 64 && !pipe_offsets_fit(BM, BN, lda, ldb)) return hipErrorInvalidValue;
        const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
        const int wg_per_cu = p.out_bf16 && p.S == 1 && !p.atomic ? PipeLds<BM, BN, NS, 1, BK * 2>::WG_PER_CU
                                                                    : PipeLds<BM, BN, NS, 0, BK * 2>::WG_PER_CU;
        const int group_m = p.group_m > 0 ? p.group_m : walk_group_m(tiles_m, tiles_n, BM, BN, wg_per_cu);
        dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)p.S), block(64 * WM * WN);
        if (p.atomic)  // free-order twin only
            hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, NS, 3, 0, BK>), grid, block, 0, stream, A, lda,
                               B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m, RedArgs{});
        else if (p.S > 1)
            hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, NS, 2, 0, BK>), grid, block, 0, stream, A, lda,
                               B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m, RedArgs{});
        else if (p.out_bf16)
            hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, NS, 1, 0, BK>), grid, block, 0, stream, A, lda,
                               B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m, RedArgs{});
        else
            hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, NS, 0, 0, BK>), grid, block, 0, stream, A, lda,
                               B, ldb, C, ldc, ws, M, N, p.cuts, tiles_m, tiles_n, group_m, RedArgs{});
        return hipGetLastError();
    }
};

template <>
struct TileLauncher<0> {
    template <int INSTR, int BM, int BN, int BK, int WM, int WN, int NS>
    static hipError_t run(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                          const uint16_t* B, int64_t ldb, void* C, int64_t ldc, float* ws, hipStream_t stream)
    {
        dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)p.S);
        dim3 block(64 * WM * WN);
        if (p.atomic)
            hipLaunchKernelGGL((gemm_bf16_kernel<INSTR, BM, BN, BK, WM, WN, false, 2>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts);
        else if (p.S > 1)
            hipLaunchKernelGGL((gemm_bf16_kernel<INSTR, BM, BN, BK, WM, WN, false, 1>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts);
        else if (p.out_bf16)
            hipLaunchKernelGGL((gemm_bf16_kernel<INSTR, BM, BN, BK, WM, WN, true, 0>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts);
        else
            hipLaunchKernelGGL((gemm_bf16_kernel<INSTR, BM, BN, BK, WM, WN, false, 0>), grid, block, 0,
                               stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts);
        return hipGetLastError();
    }
};

template <bool OUT_BF16>
hipError_t launch_combine(int S, int64_t M, int64_t N, const float* ws, void* C, int64_t ldc,
                          hipStream_t stream)
{
    const int64_t total = M * N;
    dim3 grid((unsigned)((total + 255) / 256)), block(256);
#define BG_COMBINE_CASE(NS)                                                                        \
    case NS:                                                                                       \
        hipLaunchKernelGGL((splitk_combine_kernel<NS, OUT_BF16>), grid, block, 0, stream, ws, S, M, \
                           N, C, ldc);                                                             \
        break;
    switch (S) {
        BG_COMBINE_CASE(2)
        BG_COMBINE_CASE(3)
        BG_COMBINE_CASE(4)
        BG_COMBINE_CASE(5)
        BG_COMBINE_CASE(6)
        BG_COMBINE_CASE(7)
        BG_COMBINE_CASE(8)
        BG_COMBINE_CASE(16)
    default:
        hipLaunchKernelGGL((splitk_combine_kernel<0, OUT_BF16>), grid, block, 0, stream, ws, S, M, N,
                           C, ldc);
    }
#undef BG_COMBINE_CASE
    return hipGetLastError();
}

// C[m][0..N) = 0 for every row, with the row stride ldc (a kernel rather
// than a memset so that the pitch is honoured).
__global__ __launch_bounds__(256) void zero_rows_kernel(float* __restrict__ C, int64_t M, int64_t N, int64_t ldc)
{
    const int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256)
        C[(i / N) * ldc + i % N] = 0.0f;
}

}  // namespace gemm_impl

using namespace gemm_impl;

hipError_t launch_zero_rows(float* C, int64_t M, int64_t N, int64_t ldc, hipStream_t stream)
{
    const int64_t total = M * N;
    int64_t blocks = (total + 255) / 256;
    blocks = blocks < 4096 ? blocks : 4096;
    hipLaunchKernelGGL(zero_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, M, N, ldc);
    return hipGetLastError();
}

// The tile shapes compiled in: (instruction, BM, BN, BK, waves_m, waves_n,
// load path: 0 registers, 1 direct-to-LDS, 2 pipelined direct-to-LDS, LDS
// stages of the pipelined path; the other paths double-buffer).  The first
// entry of a shape is its default stage count.
#define BG_GEMM_TILES(X)                                            \
    X(BG_MFMA_F32_32X32X16_BF16, 320, 256, 64, 2, 4, 2, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 320, 64, 4, 2, 2, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 192, 128, 64, 2, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 128, 64, 2, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 64, 64, 2, 2, 2, 4)           \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 64, 64, 2, 2, 2, 6)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 64, 64, 1, 2, 2, 6)            \
    X(BG_MFMA_F32_32X32X16_BF16, 320, 256, 32, 2, 4, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 320, 32, 4, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 256, 32, 2, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 256, 32, 2, 4, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 128, 32, 2, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 128, 32, 2, 2, 2, 6)          \
    X(BG_MFMA_F32_32X32X16_BF16, 192, 128, 32, 2, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 192, 128, 32, 2, 2, 2, 6)          \
    X(BG_MFMA_F32_32X32X16_BF16, 192, 256, 32, 2, 4, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 128, 32, 2, 2, 2, 4)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 128, 32, 2, 2, 2, 5)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 128, 32, 2, 2, 2, 8)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 64, 32, 2, 2, 2, 4)           \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 64, 32, 2, 2, 2, 8)           \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 128, 32, 2, 2, 2, 4)           \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 128, 32, 2, 2, 2, 8)           \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 64, 32, 2, 2, 2, 4)            \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 64, 32, 2, 2, 2, 8)            \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 64, 32, 2, 2, 2, 12)           \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 128, 32, 1, 4, 2, 4)           \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 128, 32, 1, 4, 2, 8)           \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 64, 32, 1, 2, 2, 4)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 64, 32, 1, 2, 2, 8)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 64, 32, 1, 2, 2, 12)           \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 32, 32, 1, 1, 2, 4)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 32, 32, 1, 1, 2, 8)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 32, 32, 1, 1, 2, 16)           \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 256, 64, 2, 2, 1, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 256, 64, 2, 4, 1, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 256, 128, 64, 2, 2, 1, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 256, 64, 2, 2, 1, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 128, 64, 2, 2, 1, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 128, 128, 64, 2, 2, 0, 2)          \
    X(BG_MFMA_F32_32X32X16_BF16, 64, 64, 64, 2, 2, 0, 2)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 64, 64, 1, 2, 0, 2)            \
    X(BG_MFMA_F32_32X32X16_BF16, 32, 32, 64, 1, 1, 0, 2)            \
    X(BG_MFMA_F32_16X16X32_BF16, 256, 256, 64, 2, 2, 1, 2)          \
    X(BG_MFMA_F32_16X16X32_BF16, 256, 128, 64, 2, 2, 1, 2)          \
    X(BG_MFMA_F32_16X16X32_BF16, 128, 128, 64, 2, 2, 0, 2)          \
    X(BG_MFMA_F32_16X16X32_BF16, 64, 64, 64, 2, 2, 0, 2)            \
    X(BG_MFMA_F32_16X16X32_BF16, 32, 32, 64, 1, 1, 0, 2)            \
    X(BG_MFMA_F32_16X16X32_BF16, 16, 32, 64, 1, 2, 0, 2)

// stages == 0 takes the first compiled entry of the shape
bool gemm_bf16_has_tile(int mfma, int bm, int bn, int bk, int waves_m, int waves_n, int direct, int stages)
{
#define BG_HAS(I, BM_, BN_, BK_, WM_, WN_, D_, NS_)                                                 \
    if (mfma == I && bm == BM_ && bn == BN_ && bk == BK_ && waves_m == WM_ && waves_n == WN_ &&      \
        direct == D_ && (stages == 0 || stages == NS_))                                              \
        return true;
    BG_GEMM_TILES(BG_HAS)
#undef BG_HAS
    return false;
}

// The (other splits, last split) tile pairs compiled in: the k tile depth
// both shapes share, then BM, BN, waves_m, waves_n, stages of each
// (pipelined path, 32x32x16).  The first entry of a pair of shapes is its
// default stage count.
#define BG_GEMM_DUAL_TILES(X)                        \
    X(32, 256, 256, 2, 2, 4, 64, 64, 2, 2, 8)        \
    X(32, 256, 256, 2, 2, 4, 128, 64, 2, 2, 4)       \
    X(32, 256, 128, 2, 2, 4, 64, 64, 2, 2, 8)        \
    X(32, 192, 128, 2, 2, 4, 64, 64, 2, 2, 8)        \
    X(32, 128, 128, 2, 2, 4, 64, 64, 2, 2, 8)        \
    X(32, 256, 256, 2, 4, 4, 128, 64, 4, 2, 8)       \
    X(32, 256, 256, 2, 4, 4, 64, 128, 2, 4, 8)       \
    X(64, 256, 256, 2, 4, 2, 128, 64, 4, 2, 4)       \
    X(64, 128, 128, 2, 2, 4, 64, 64, 2, 2, 6)        \
    X(64, 128, 128, 2, 2, 4, 128, 64, 2, 2, 4)

bool gemm_bf16_has_dual_tile(int bm, int bn, int bk, int waves_m, int waves_n, int stages, int bm2, int bn2,
                             int waves_m2, int waves_n2, int stages2)
{
#define BG_DHAS(BK_, BM_, BN_, WM_, WN_, NS_, BM2_, BN2_, WM2_, WN2_, NS2_)                                          \
    if (bk == BK_ && bm == BM_ && bn == BN_ && waves_m == WM_ && waves_n == WN_ && (stages == 0 || stages == NS_) &&  \
        bm2 == BM2_ && bn2 == BN2_ && waves_m2 == WM2_ && waves_n2 == WN2_ && (stages2 == 0 || stages2 == NS2_))       \
        return true;
    BG_GEMM_DUAL_TILES(BG_DHAS)
#undef BG_DHAS
    return false;
}

template <int BK, int BM, int BN, int WM, int WN, int NS, int BM2, int BN2, int WM2, int WN2, int NS2>
static hipError_t launch_dual(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                              const uint16_t* B, int64_t ldb, void* C, int64_t ldc, float* ws, hipStream_t stream)
{
    using L = DualLds<BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, BK>;
    constexpr int PER_CU = (160 * 1024) / L::BYTES;
    if (BK == 64 && ((NS == 2 && !pipe_offsets_fit(BM, BN, lda, ldb)) || (NS2 == 2 && !pipe_offsets_fit(BM2, BN2, lda, ldb))))
        return hipErrorInvalidValue;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int tiles_m2 = (int)((M + BM2 - 1) / BM2), tiles_n2 = (int)((N + BN2 - 1) / BN2);
    const int group_m = p.group_m > 0 ? p.group_m : walk_group_m(tiles_m, tiles_n, BM, BN, PER_CU);
    const int group_m2 = p.group_m > 0 ? p.group_m : walk_group_m(tiles_m2, tiles_n2, BM2, BN2, PER_CU);
    const int64_t wgs = (int64_t)tiles_m * tiles_n * (p.S - 1) + (int64_t)tiles_m2 * tiles_n2;
    if (p.S < 2 || wgs > 0x7fffffff) return hipErrorInvalidValue;
    if (p.atomic)  // free-order twin only
        hipLaunchKernelGGL((gemm_bf16_pipe_dual_kernel<BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, 3, BK>),
                           dim3((unsigned)wgs), dim3(64 * WM * WN), 0, stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts,
                           p.S, tiles_m, tiles_n, group_m, tiles_m2, tiles_n2, group_m2, p.last_first ? 1 : 0);
    else
        hipLaunchKernelGGL((gemm_bf16_pipe_dual_kernel<BM, BN, WM, WN, NS, BM2, BN2, WM2, WN2, NS2, 2, BK>),
                           dim3((unsigned)wgs), dim3(64 * WM * WN), 0, stream, A, lda, B, ldb, C, ldc, ws, M, N, p.cuts,
                           p.S, tiles_m, tiles_n, group_m, tiles_m2, tiles_n2, group_m2, p.last_first ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const GemmPlan& p, int64_t M, int64_t N, int64_t K, const uint16_t* A,
                            int64_t lda, const uint16_t* B, int64_t ldb, void* C, int64_t ldc, float* ws,
                            hipStream_t stream)
{
    (void)K;
    hipError_t err = hipErrorInvalidValue;
    bool found = false;
#define BG_LAUNCH(I, BM_, BN_, BK_, WM_, WN_, D_, NS_)                                                  \
    if (!found && p.mfma == I && p.bm == BM_ && p.bn == BN_ && p.bk == BK_ && p.waves_m == WM_ &&      \
        p.waves_n == WN_ && p.direct == D_ && (p.stages == 0 || p.stages == NS_)) {                    \
        found = true;                                                                                    \
        err = TileLauncher<D_>::template run<I, BM_, BN_, BK_, WM_, WN_, NS_>(p, M, N, A, lda, B, ldb, C, ldc, ws, stream); \
    }
    if (p.bm2) {
#define BG_DLAUNCH(BK_, BM_, BN_, WM_, WN_, NS_, BM2_, BN2_, WM2_, WN2_, NS2_)                                   \
        if (!found && p.bk == BK_ && p.bm == BM_ && p.bn == BN_ && p.waves_m == WM_ && p.waves_n == WN_ &&       \
            (p.stages == 0 || p.stages == NS_) && p.bm2 == BM2_ && p.bn2 == BN2_ && p.waves_m2 == WM2_ &&          \
            p.waves_n2 == WN2_ && (p.stages2 == 0 || p.stages2 == NS2_)) {                                       \
            found = true;                                                                                          \
            err = launch_dual<BK_, BM_, BN_, WM_, WN_, NS_, BM2_, BN2_, WM2_, WN2_, NS2_>(p, M, N, A, lda, B, ldb, C, \
                                                                                        ldc, ws, stream);          \
        }
        BG_GEMM_DUAL_TILES(BG_DLAUNCH)
#undef BG_DLAUNCH
    } else {
        BG_GEMM_TILES(BG_LAUNCH)
    }
#undef BG_LAUNCH
    if (!found || err != hipSuccess) return found ? err : hipErrorInvalidValue;
    if (p.S > 1 && !p.atomic) {
        if (p.out_bf16) return launch_combine<true>(p.S, M, N, ws, C, ldc, stream);
        return launch_combine<false>(p.S, M, N, ws, C, ldc, stream);
    }
    return hipSuccess;
}

// Tiles built with the fused reductions (32x32x16, pipelined path): BM, BN,
// BK, waves_m, waves_n, stages -- the large-output tile (64-deep, and
// 32-deep for leading dimensions too large for its copy offsets), a
// mid-size tile and the small-M tile.
#define BG_GEMM_RED_TILES(X)  \
    X(320, 256, 64, 2, 4, 2)  \
    X(320, 256, 32, 2, 4, 4)  \
    X(256, 128, 32, 2, 2, 4)  \
    X(64, 64, 32, 2, 2, 8)

bool gemm_bf16_red_has_tile(int bm, int bn, int bk, int waves_m, int waves_n, int stages)
{
#define BG_RHAS(BM_, BN_, BK_, WM_, WN_, NS_)                                                      \
    if (bm == BM_ && bn == BN_ && bk == BK_ && waves_m == WM_ && waves_n == WN_ &&               \
        (stages == 0 || stages == NS_))                                                          \
        return true;
    BG_GEMM_RED_TILES(BG_RHAS)
#undef BG_RHAS
    return false;
}

template <int BM, int BN, int BK, int WM, int WN, int NS, int OUT, int RED>
static hipError_t launch_red_tile(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                                  const uint16_t* B, int64_t ldb, void* C, int64_t ldc, hipStream_t stream)
{
    if (BK == 64 && !pipe_offsets_fit(BM, BN, lda, ldb)) return hipErrorInvalidValue;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int group_m =
        p.group_m > 0 ? p.group_m
                      : walk_group_m(tiles_m, tiles_n, BM, BN, PipeLds<BM, BN, NS, OUT, BK * 2>::WG_PER_CU);
    dim3 grid((unsigned)(tiles_m * tiles_n)), block(64 * WM * WN);
    hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, NS, OUT, RED, BK>), grid, block, 0, stream, A, lda, B,
                       ldb, C, ldc, (float*)nullptr, M, N, p.cuts, tiles_m, tiles_n, group_m, p.red_args);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16_reduce(const GemmPlan& p, int64_t M, int64_t N, const uint16_t* A, int64_t lda,
                                   const uint16_t* B, int64_t ldb, void* C, int64_t ldc, hipStream_t stream)
{
    if (p.S != 1 || (p.red != 1 && p.red != 2) || p.mfma != BG_MFMA_F32_32X32X16_BF16) return hipErrorInvalidValue;
#define BG_RLAUNCH(BM_, BN_, BK_, WM_, WN_, NS_)                                                                   \
    if (p.bm == BM_ && p.bn == BN_ && p.bk == BK_ && p.waves_m == WM_ && p.waves_n == WN_ &&                       \
        (p.stages == 0 || p.stages == NS_)) {                                                                     \
        if (p.out_bf16)                                                                                           \
            return p.red == 1                                                                                     \
                       ? launch_red_tile<BM_, BN_, BK_, WM_, WN_, NS_, 1, 1>(p, M, N, A, lda, B, ldb, C, ldc, stream) \
                       : launch_red_tile<BM_, BN_, BK_, WM_, WN_, NS_, 1, 2>(p, M, N, A, lda, B, ldb, C, ldc, stream); \
        return p.red == 1                                                                                         \
                   ? launch_red_tile<BM_, BN_, BK_, WM_, WN_, NS_, 0, 1>(p, M, N, A, lda, B, ldb, C, ldc, stream)     \
                   : launch_red_tile<BM_, BN_, BK_, WM_, WN_, NS_, 0, 2>(p, M, N, A, lda, B, ldb, C, ldc, stream);    \
    }
    BG_GEMM_RED_TILES(BG_RLAUNCH)
#undef BG_RLAUNCH
    return hipErrorInvalidValue;
}

// The free-order twin with two interleaved accumulator chains per output
// (bench only): the 128x128 tile with 64-deep k tiles in a ring of four, the
// same main loop as that tile's order-fixed kernel, fp32 C.
hipError_t launch_gemm_bf16_two_chains(int64_t M, int64_t N, int64_t K, const uint16_t* A, int64_t lda,
                                       const uint16_t* B, int64_t ldb, float* C, int64_t ldc, hipStream_t stream)
{
    constexpr int BM = 128, BN = 128, WM = 2, WN = 2, NS = 4, BK = 64;
    if (!pipe_offsets_fit(BM, BN, lda, ldb)) return hipErrorInvalidValue;
    const int tiles_m = (int)((M + BM - 1) / BM), tiles_n = (int)((N + BN - 1) / BN);
    const int group_m = walk_group_m(tiles_m, tiles_n, BM, BN, PipeLds<BM, BN, NS, 0, BK * 2>::WG_PER_CU);
    Cuts cuts{};
    cuts.c[0] = 0, cuts.c[1] = K;
    hipLaunchKernelGGL((gemm_impl::gemm_bf16_pipe_kernel<BM, BN, WM, WN, NS, 4, 0, BK>), dim3(tiles_m * tiles_n),
                       dim3(64 * WM * WN), 0, stream, A, lda, B, ldb, (void*)C, ldc, (float*)nullptr, M, N, cuts,
                       tiles_m, tiles_n, group_m, RedArgs{});
    return hipGetLastError();
}

}  // namespace bg
