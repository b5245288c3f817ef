// bg_pipe.h -- device helpers shared by the pipelined GEMM kernels (bf16 and
// W8A8) of libbitgemm: the workgroup-to-tile walk, the direct global-to-LDS
// copy issued outside the compiler's view, the explicit copy waits, and the
// swizzle of an output tile staged in LDS.  gfx950 only.
#pragma once

#include "bg_internal.h"

namespace bg {

// Workgroup -> output tile.  Workgroups are handed to the 8 XCDs in turn, so
// consecutive ids land on different L2s; renumber them so that each XCD gets
// one contiguous run of tiles, then walk that run GROUP_M tile-rows at a time
// (column-major inside a group) so that neighbours share A rows and B columns.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int group_m, int& tm, int& tn)
{
    const int T = tiles_m * tiles_n;
    const int q = T / 8, r = T % 8;
    const int x = b % 8, j = b / 8;
    const int bb = x * q + (x < r ? x : r) + j;  // a bijection on [0, T)
    const int per_group = group_m * tiles_n;
    const int g = bb / per_group;
    const int first_m = g * group_m;
    const int gsize = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int in = bb - g * per_group;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

// Default group height of that walk (host side).  One XCD (32 CUs on gfx950)
// runs c = 32 * wg_per_cu of its tiles at a time, about gm tile rows by c / gm
// tile columns, and its L2 fetches gm * bm rows of A plus (c / gm) * bn rows
// of B for them; gm = sqrt(c * bn / bm) makes that smallest.
inline int walk_group_m(int tiles_m, int tiles_n, int bm, int bn, int wg_per_cu)
{
    const long long per_xcd = ((long long)tiles_m * tiles_n + 7) / 8;
    long long c = 32LL * (wg_per_cu < 1 ? 1 : wg_per_cu);
    if (c > per_xcd) c = per_xcd;
    int g = (int)(__builtin_sqrt((double)c * bn / bm) + 0.5);
    if (g > tiles_m) g = tiles_m;
    return g < 1 ? 1 : g;
}

// 16 bytes from global memory into LDS at byte address lds_addr + 16 * lane
// (global_load_lds_dwordx4; M0 holds the LDS address and is restored).  It is
// issued as inline assembly so that the compiler, which cannot place an LDS
// DMA among its LDS reads, does not drain every read before each MFMA; the
// copies are waited for with explicit vmcnt waits.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds_addr)
{
    // the LDS address is the same for every lane; make that visible to the
    // compiler so that it sits in a scalar register
    lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds_addr)
        : "memory");
}

// The same copy addressed as a 64-bit scalar base plus a 32-bit byte offset
// per lane (the global instruction's scalar-base form), so that a lane keeps
// one register per copy instead of a pointer pair: the base walks k in
// scalar registers, the offsets stay fixed for the whole walk.
__device__ __forceinline__ void dma16_off(const void* base, uint32_t off, uint32_t lds_addr)
{
    lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds_addr)
        : "memory");
}

// s_waitcnt lgkmcnt(0), other counters untouched: this wave's LDS reads and
// writes are complete
__device__ __forceinline__ void wait_lgkmcnt0()
{
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// s_waitcnt vmcnt(N), other counters untouched
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt holds 0..63");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// wait until at most `newer` turns of LOADS copies each are outstanding
// (newer <= MAXN; a larger value waits for more than needed, never less)
template <int LOADS, int MAXN>
__device__ __forceinline__ void wait_turns(int newer)
{
    if constexpr (MAXN >= 1) {
        if (newer >= MAXN) {
            wait_vmcnt<MAXN * LOADS>();
            return;
        }
        wait_turns<LOADS, MAXN - 1>(newer);
    } else {
        wait_vmcnt<0>();
    }
}

// Staged bf16 C rows hold CHR 16-byte chunks; chunk ch of row m is stored at
// position ch ^ (m & mask) inside its row (within the leading power of two of
// chunks, and within the trailing eight), so that the writes of 16
// consecutive rows to one column chunk land in distinct bank groups.
template <int CHR>
__device__ __forceinline__ int c_swizzle(int ch, int m)
{
    static_assert(CHR == 4 || CHR == 8 || CHR == 16 || CHR == 24 || CHR == 32 || CHR == 40,
                  "staged row widths: 32, 64, 128, 192, 256 or 320 columns");
    if constexpr (CHR == 40) return ch < 32 ? ch ^ (m & 31) : ch ^ (m & 7);
    else if constexpr (CHR == 24) return ch < 16 ? ch ^ (m & 15) : ch ^ (m & 7);
    else return ch ^ (m & (CHR - 1));
}

// LDS a pipelined kernel uses (NS stages of a k tile of ROW_BYTES per row of
// A and B; a bf16 output tile staged when OUT == 1), and the waves per SIMD
// that leaves room for
template <int BM, int BN, int NS, int OUT, int ROW_BYTES = 64>
struct PipeLds {
    static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
    static constexpr int PIPE = NS * STAGE_BYTES, EPI = OUT == 1 ? BM * BN * 2 : 0;
    static constexpr int BYTES = PIPE > EPI ? PIPE : EPI;
    static constexpr int WG_PER_CU = (160 * 1024) / BYTES;
};
template <int BM, int BN, int WM, int WN, int NS, int OUT, int ROW_BYTES = 64>
struct PipeOcc {
    static constexpr int W = PipeLds<BM, BN, NS, OUT, ROW_BYTES>::WG_PER_CU * WM * WN / 4;
    static constexpr int WAVES_PER_EU = W < 1 ? 1 : W;
};

}  // namespace bg
