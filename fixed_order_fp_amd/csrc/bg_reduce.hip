// bg_reduce.hip -- fixed-order row and column reductions (sum and sum of
// squares) for gfx950, and their free-order twins for the bench.
//
// Order ("Taming Bitwise Behavior", 3.1 and 5.1): the reduced axis is cut
// into leaves of 32 consecutive elements; each leaf is folded by one lane in
// index order with no +0 seed (s = x0; s = s + xi; q = x0*x0; q = fma(xi, xi,
// q)); the leaves are then combined by a balanced tree over the leaf index,
// neighbours first (count-up offsets 1, 2, 4, ...), an odd node carried up.
// Node i of level l covers the leaves [i 2^l, (i+1) 2^l), so any aligned run
// of 2^l leaves is an exact subtree: a workgroup folds such a run, and when an
// axis needs several workgroups their subtree roots go to a workspace and a
// second kernel applies the upper levels of the same tree.  Nothing depends
// on the number of compute units, and nothing uses atomics.
//
// Row axis: a workgroup of 4 waves owns 256 leaves (8192 elements) of one
// row; each lane loads its own leaf (128 B of fp32 or 64 B of bf16) with
// 16-byte vector loads -- consecutive lanes read consecutive 128 B lines, so a
// wave's loads cover whole lines with nothing to stage or transpose -- and
// folds it in registers.  The 64 leaves of a wave are combined with DPP
// row shifts (offsets 1, 2, 4, 8, the right node added to the left one in
// its own lane) and the four row roots read back as (r0 + r1) + (r2 + r3).
// Column axis: a lane covers 16 adjacent bytes of a row (8 bf16 or 4 fp32
// columns), a wave folds one leaf (32 rows) at a time with all of the leaf's
// row loads in flight, and the waves of a workgroup hold consecutive leaves,
// combined through LDS.
#include <type_traits>

#include "bg_internal.h"

namespace bg {

namespace reduce_impl {

constexpr int kLeaf = 32;

// The count-up tree over one wave's 64 nodes (lane l holds node l of this
// level run); n_valid = how many of the 64 exist.  Lane 0 ends with the root.
__device__ __forceinline__ float wave_tree(float v, int lane, int n_valid)
{
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_down(v, d, 64);
        if ((lane & (2 * d - 1)) == 0 && lane + d < n_valid) v = v + o;
    }
    return v;
}

// The same count-up tree for a wave whose 64 nodes all exist, with DPP row
// shifts: after the step of offset d, lane l with l = -1 mod 2d holds the node
// covering lanes (l - 2d, l], computed as left + right.  Offsets 16 and 32
// cross DPP rows; they are taken from the four row roots (lanes 15, 31, 47,
// 63) read into scalars.  Every lane returns the root.
__device__ __forceinline__ float wave_tree_full(float v)
{
    const int lane = threadIdx.x & 63;
    float o;
    o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, false));  // row_shr:1
    if ((lane & 1) == 1) v = o + v;
    o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xf, 0xf, false));  // row_shr:2
    if ((lane & 3) == 3) v = o + v;
    o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xf, 0xf, false));  // row_shr:4
    if ((lane & 7) == 7) v = o + v;
    o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xf, 0xf, false));  // row_shr:8
    if ((lane & 15) == 15) v = o + v;
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 15));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 47));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return (r0 + r1) + (r2 + r3);
}

// element i of 8 bf16 packed in a u32x4 (little endian: even elements in the
// low halves)
__device__ __forceinline__ float bf16_lane(const u32x4& v, int i)
{
    const uint32_t w = v[i / 2];
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <bool FUSED>
__device__ __forceinline__ void fold_step(float x, float& s, float& q)
{
    s = s + x;
    if constexpr (FUSED) q = __builtin_fmaf(x, x, q);
    else {
        const float xx = x * x;
        q = q + xx;
    }
}

// Fold one whole leaf (32 elements at p, 16-byte aligned) in index order.
template <typename T, bool FUSED>
__device__ __forceinline__ void fold_leaf_vec(const T* p, float& s, float& q)
{
    if constexpr (std::is_same<T, float>::value) {
        u32x4 c[8];
#pragma unroll
        for (int i = 0; i < 8; i++) c[i] = *(const u32x4*)(p + 4 * i);
        s = __uint_as_float(c[0][0]);
        q = s * s;
#pragma unroll
        for (int i = 1; i < kLeaf; i++) fold_step<FUSED>(__uint_as_float(c[i / 4][i % 4]), s, q);
    } else {
        u32x4 c[4];
#pragma unroll
        for (int i = 0; i < 4; i++) c[i] = *(const u32x4*)(p + 8 * i);
        s = bf16_lane(c[0], 0);
        q = s * s;
#pragma unroll
        for (int i = 1; i < kLeaf; i++) fold_step<FUSED>(bf16_lane(c[i / 8], i % 8), s, q);
    }
}

// Balanced tree over v[0..n), n <= N, in place: at stride d the node at i
// (a multiple of 2d) absorbs its right neighbour i + d when that node exists
// (i + d < n), which is the neighbours-first pairing with an odd last node
// carried up unchanged.  N is a compile-time bound so v stays in registers.
template <int N>
__device__ __forceinline__ float tree_upto(float* v, int n)
{
#pragma unroll
    for (int d = 1; d < N; d <<= 1)
#pragma unroll
        for (int i = 0; i + d < N; i += 2 * d)
            if (i + d < n) v[i] = v[i] + v[i + d];
    return v[0];
}

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// Fold one leaf held in registers: x[0..n) in index order, no seed.
template <bool FUSED>
__device__ __forceinline__ void fold_leaf(const float* x, int n, float& s, float& q)
{
    s = x[0];
    q = x[0] * x[0];
    for (int i = 1; i < n; i++) {
        s = s + x[i];
        if constexpr (FUSED) q = __builtin_fmaf(x[i], x[i], q);
        else {
            const float xx = x[i] * x[i];
            q = q + xx;
        }
    }
}

// ---- row axis ---------------------------------------------------------------
// One workgroup: row `row`, leaf block `blk` (256 leaves).  A full block takes
// the vector path; a short block folds element by element.
template <typename T, bool FUSED>
__global__ __launch_bounds__(256) void reduce_row_kernel(const T* __restrict__ X, int64_t ldx, int64_t cols,
                                                         float* __restrict__ out_sum, float* __restrict__ out_sq,
                                                         float* __restrict__ ws, int n_blocks)
{
    __shared__ float roots[2][4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row = blockIdx.x;
    const int blk = blockIdx.y;
    const int64_t n_leaf_row = (cols + kLeaf - 1) / kLeaf;
    const int64_t leaf0 = (int64_t)blk * 256;
    const int n_valid = (int)((n_leaf_row - leaf0) < 256 ? (n_leaf_row - leaf0) : 256);
    const T* xr = X + row * ldx;
    const int my_leaf = wave * 64 + lane;  // within the block

    float s = 0.0f, q = 0.0f;
    // the whole block present and every leaf 16-byte aligned (X 16-byte
    // aligned, ldx a multiple of 8, leaves of 32 elements)
    const bool full = (leaf0 + 256) * kLeaf <= cols;
    if (full) {
        fold_leaf_vec<T, FUSED>(xr + (leaf0 + my_leaf) * kLeaf, s, q);
        s = wave_tree_full(s);
        q = wave_tree_full(q);
    } else {
        if (my_leaf < n_valid) {
            const int64_t e0 = (leaf0 + my_leaf) * kLeaf;
            const int n = (int)((cols - e0) < kLeaf ? (cols - e0) : kLeaf);
            float x[kLeaf];
            for (int i = 0; i < n; i++) x[i] = load_elem<T>(xr + e0 + i);
            fold_leaf<FUSED>(x, n, s, q);
        }
        const int wave_valid = n_valid - wave * 64;
        s = wave_tree(s, lane, wave_valid);
        q = wave_tree(q, lane, wave_valid);
    }
    // this wave's root (leaves [64 wave, 64 wave + 64)) is in lane 0
    if (lane == 0) {
        roots[0][wave] = s;
        roots[1][wave] = q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n_waves = (n_valid + 63) / 64;
        float vs[4], vq[4];
#pragma unroll
        for (int w = 0; w < 4; w++) vs[w] = roots[0][w], vq[w] = roots[1][w];
        const float rs = tree_upto<4>(vs, n_waves), rq = tree_upto<4>(vq, n_waves);
        if (n_blocks == 1) {
            if (out_sum) out_sum[row] = rs;
            if (out_sq) out_sq[row] = rq;
        } else {
            ws[(row * n_blocks + blk) * 2] = rs;
            ws[(row * n_blocks + blk) * 2 + 1] = rq;
        }
    }
}

// Upper tree levels over the block roots of one output (n_blocks <= NB).
template <int NB>
__global__ __launch_bounds__(256) void reduce_blocks_kernel(const float* __restrict__ ws, int64_t n_out,
                                                            int n_blocks, int64_t stride_out, int64_t stride_blk,
                                                            float* __restrict__ out_sum, float* __restrict__ out_sq)
{
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n_out) return;
    float vs[NB], vq[NB];
    // every load is issued (past the last block it re-reads a valid one, never
    // used) so that all of them are in flight at once
#pragma unroll
    for (int b = 0; b < NB; b++) {
        const int64_t blk = b < n_blocks ? b : n_blocks - 1;
        vs[b] = ws[(o * stride_out + blk * stride_blk) * 2];
        vq[b] = ws[(o * stride_out + blk * stride_blk) * 2 + 1];
    }
    const float rs = tree_upto<NB>(vs, n_blocks), rq = tree_upto<NB>(vq, n_blocks);
    if (out_sum) out_sum[o] = rs;
    if (out_sq) out_sq[o] = rq;
}

hipError_t launch_blocks(const float* ws, int64_t n_out, int nb, int64_t stride_out, int64_t stride_blk,
                         float* out_sum, float* out_sq, hipStream_t stream)
{
    dim3 grid((unsigned)((n_out + 255) / 256)), block(256);
    if (nb <= 4)
        hipLaunchKernelGGL(reduce_blocks_kernel<4>, grid, block, 0, stream, ws, n_out, nb, stride_out, stride_blk,
                           out_sum, out_sq);
    else if (nb <= 16)
        hipLaunchKernelGGL(reduce_blocks_kernel<16>, grid, block, 0, stream, ws, n_out, nb, stride_out, stride_blk,
                           out_sum, out_sq);
    else
        hipLaunchKernelGGL(reduce_blocks_kernel<64>, grid, block, 0, stream, ws, n_out, nb, stride_out, stride_blk,
                           out_sum, out_sq);
    return hipGetLastError();
}

// Upper tree levels of the column axis: roots ws[blk][col] (sum, sumsq
// interleaved).  A workgroup of 4 waves takes 64 adjacent columns; wave p
// folds the aligned run of block roots [p NBP, (p+1) NBP) of each column (an
// exact subtree: one load per block covers 64 adjacent columns), and the four
// run roots are paired through LDS as the tree's top two levels.
template <int NBP>
__global__ __launch_bounds__(256) void reduce_col_blocks_kernel(const float* __restrict__ ws, int64_t cols,
                                                                int n_blocks, float* __restrict__ out_sum,
                                                                float* __restrict__ out_sq)
{
    __shared__ float part[2][4][64];
    const int lane = threadIdx.x & 63;
    const int p = threadIdx.x >> 6;
    const int64_t col = (int64_t)blockIdx.x * 64 + lane;
    const int first = p * NBP;
    const int n = n_blocks - first < NBP ? (n_blocks - first > 0 ? n_blocks - first : 0) : NBP;
    float vs[NBP], vq[NBP];
    // every load is issued (past the last block or column it re-reads a valid
    // one, never used) so that all of them are in flight at once
    const int64_t c = col < cols ? col : cols - 1;
#pragma unroll
    for (int b = 0; b < NBP; b++) vs[b] = 0.0f, vq[b] = 0.0f;
    if (out_sum) {
#pragma unroll
        for (int b = 0; b < NBP; b++) {
            const int blk = first + b < n_blocks ? first + b : n_blocks - 1;
            vs[b] = ws[(c + (int64_t)blk * cols) * 2];
        }
    }
    if (out_sq) {
#pragma unroll
        for (int b = 0; b < NBP; b++) {
            const int blk = first + b < n_blocks ? first + b : n_blocks - 1;
            vq[b] = ws[(c + (int64_t)blk * cols) * 2 + 1];
        }
    }
    part[0][p][lane] = n ? tree_upto<NBP>(vs, n) : 0.0f;
    part[1][p][lane] = n ? tree_upto<NBP>(vq, n) : 0.0f;
    __syncthreads();
    if (p == 0 && col < cols) {
        const int n_parts = (n_blocks + NBP - 1) / NBP;
        float rs[4], rq[4];
#pragma unroll
        for (int k = 0; k < 4; k++) rs[k] = part[0][k][lane], rq[k] = part[1][k][lane];
        if (out_sum) out_sum[col] = tree_upto<4>(rs, n_parts);
        if (out_sq) out_sq[col] = tree_upto<4>(rq, n_parts);
    }
}

hipError_t launch_col_blocks(const float* ws, int64_t cols, int nb, float* out_sum, float* out_sq,
                             hipStream_t stream)
{
    dim3 grid((unsigned)((cols + 63) / 64)), block(256);
    if (nb <= 4)
        hipLaunchKernelGGL(reduce_col_blocks_kernel<1>, grid, block, 0, stream, ws, cols, nb, out_sum, out_sq);
    else if (nb <= 16)
        hipLaunchKernelGGL(reduce_col_blocks_kernel<4>, grid, block, 0, stream, ws, cols, nb, out_sum, out_sq);
    else
        hipLaunchKernelGGL(reduce_col_blocks_kernel<16>, grid, block, 0, stream, ws, cols, nb, out_sum, out_sq);
    return hipGetLastError();
}

// ---- leaf sums written by another kernel (the GEMM epilogue) ----------------
// ws_sum / ws_sq hold one fp32 leaf node per leaf and output, [leaf][n_out].
// A workgroup of 16 waves takes 64 adjacent outputs; wave p folds the aligned
// runs of 32 leaves p and p + 16 (exact level-5 subtrees of the balanced tree;
// at most 32 runs: 1024 leaves, one round for up to 512), with the loads of
// both outputs in flight at once, and the run roots are paired through LDS as
// the tree's top levels.
__global__ __launch_bounds__(1024) void leaf_tree_kernel(const float* __restrict__ ws_sum,
                                                         const float* __restrict__ ws_sq, int64_t n_out,
                                                         int n_leaf, float* __restrict__ out_sum,
                                                         float* __restrict__ out_sq)
{
    __shared__ float part[2][32][64];
    const int lane = threadIdx.x & 63;
    const int p = threadIdx.x >> 6;
    const int64_t o = (int64_t)blockIdx.x * 64 + lane;
    const int64_t oc = o < n_out ? o : n_out - 1;  // past the last output: a valid re-read, never stored
    const int n_runs = (n_leaf + 31) / 32;
    for (int r = p; r < n_runs; r += 16) {
        const int first = r * 32;
        const int n = n_leaf - first < 32 ? n_leaf - first : 32;
        float vs[32], vq[32];
#pragma unroll
        for (int b = 0; b < 32; b++) {
            const int64_t at = (int64_t)(first + (b < n ? b : n - 1)) * n_out + oc;
            vs[b] = ws_sum ? ws_sum[at] : 0.0f;
            vq[b] = ws_sq ? ws_sq[at] : 0.0f;
        }
        part[0][r][lane] = tree_upto<32>(vs, n);
        part[1][r][lane] = tree_upto<32>(vq, n);
    }
    __syncthreads();
    if (p == 0 && o < n_out) {
        float rs[32], rq[32];
#pragma unroll
        for (int r = 0; r < 32; r++) {
            rs[r] = r < n_runs ? part[0][r][lane] : 0.0f;
            rq[r] = r < n_runs ? part[1][r][lane] : 0.0f;
        }
        if (out_sum) out_sum[o] = tree_upto<32>(rs, n_runs);
        if (out_sq) out_sq[o] = tree_upto<32>(rq, n_runs);
    }
}

// ---- column axis ------------------------------------------------------------
// A workgroup of 4 waves covers 64 * CPL adjacent columns (CPL * sizeof(T) =
// 16 or 8 bytes per lane) and 4 * LPWAVE consecutive leaves starting at leaf
// block `blk`; wave w folds leaves [w LPWAVE, (w+1) LPWAVE) of that run one
// after the other and pairs them into its node; the four wave nodes are then
// paired through LDS.
//
// One lane's piece of one row.  Every element is read once and each load
// instruction covers whole contiguous row segments, so the loads are
// streaming (non-temporal): 5-8 % faster here.  The row axis keeps ordinary
// loads: its lanes read a leaf as several 16-byte pieces of the same lines,
// which then come back from the cache (streaming loads made it 1.5-2.4x
// slower).
template <typename T, int CPL>
__device__ __forceinline__ void load_row_vec(const T* p, float* x)
{
    if constexpr (std::is_same<T, float>::value) {
        static_assert(CPL == 4, "fp32 rows are read 16 bytes per lane");
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
#pragma unroll
        for (int c = 0; c < 4; c++) x[c] = __uint_as_float(v[c]);
    } else if constexpr (CPL == 8) {
        const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
#pragma unroll
        for (int c = 0; c < 8; c++) x[c] = bf16_lane(v, c);
    } else {
        static_assert(CPL == 4, "bf16 rows are read 16 or 8 bytes per lane");
        const unsigned long long w = __builtin_nontemporal_load((const unsigned long long*)p);
        const uint32_t lo = (uint32_t)w, hi = (uint32_t)(w >> 32);
        x[0] = __uint_as_float(lo << 16);
        x[1] = __uint_as_float(lo & 0xffff0000u);
        x[2] = __uint_as_float(hi << 16);
        x[3] = __uint_as_float(hi & 0xffff0000u);
    }
}

template <typename T, int CPL, int LPWAVE, bool FUSED>
__global__ __launch_bounds__(256) void reduce_col_kernel(const T* __restrict__ X, int64_t ldx, int64_t rows,
                                                         int64_t cols, float* __restrict__ ws,
                                                         float* __restrict__ out_sum, float* __restrict__ out_sq,
                                                         int n_blocks)
{
    constexpr int LPW = 4 * LPWAVE;
    __shared__ float part[2][4][64 * CPL];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * 64 * CPL + lane * CPL;
    const int blk = blockIdx.y;
    const int64_t n_leaf = (rows + kLeaf - 1) / kLeaf;
    const int64_t wleaf0 = (int64_t)blk * LPW + wave * LPWAVE;  // this wave's first leaf
    const bool vec = col0 + CPL <= cols;

    float ls[LPWAVE][CPL], lq[LPWAVE][CPL];
    int n_mine = 0;  // leaves of this wave that exist
#pragma unroll
    for (int l = 0; l < LPWAVE; l++) {
        const int64_t leaf = wleaf0 + l;
        if (leaf >= n_leaf) break;
        n_mine = l + 1;
        const int64_t r0 = leaf * kLeaf;
        const int n = (int)((rows - r0) < kLeaf ? (rows - r0) : kLeaf);
        float s[CPL], q[CPL];
        if (n == kLeaf && vec) {
            // the whole leaf: 32 independent row loads, folded in row order
            float x[kLeaf][CPL];
#pragma unroll
            for (int i = 0; i < kLeaf; i++) load_row_vec<T, CPL>(X + (r0 + i) * ldx + col0, x[i]);
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                s[c] = x[0][c];
                q[c] = x[0][c] * x[0][c];
            }
#pragma unroll
            for (int i = 1; i < kLeaf; i++)
#pragma unroll
                for (int c = 0; c < CPL; c++) fold_step<FUSED>(x[i][c], s[c], q[c]);
        } else {
            // a short leaf or the ragged right edge, element by element
            for (int i = 0; i < n; i++) {
                const T* p = X + (r0 + i) * ldx + col0;
#pragma unroll
                for (int c = 0; c < CPL; c++) {
                    const float x = (col0 + c < cols) ? load_elem<T>(p + c) : 0.0f;
                    if (i == 0) {
                        s[c] = x;
                        q[c] = x * x;
                    } else {
                        fold_step<FUSED>(x, s[c], q[c]);
                    }
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CPL; c++) ls[l][c] = s[c], lq[l][c] = q[c];
    }
    // this wave's leaves -> one node (balanced, neighbours first, odd carried)
    float ws_[CPL], wq_[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) {
        float vs[LPWAVE], vq[LPWAVE];
#pragma unroll
        for (int l = 0; l < LPWAVE; l++) vs[l] = ls[l][c], vq[l] = lq[l][c];
        ws_[c] = n_mine ? tree_upto<LPWAVE>(vs, n_mine) : 0.0f;
        wq_[c] = n_mine ? tree_upto<LPWAVE>(vq, n_mine) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < CPL; c++) {
        part[0][wave][lane * CPL + c] = ws_[c];
        part[1][wave][lane * CPL + c] = wq_[c];
    }
    __syncthreads();
    // the workgroup's waves -> one node; waves with no leaf do not exist
    const int64_t blk_leaf0 = (int64_t)blk * LPW;
    const int64_t left = (n_leaf - blk_leaf0 + LPWAVE - 1) / LPWAVE;
    const int n_waves = (int)(left < 4 ? left : 4);
    for (int idx = threadIdx.x; idx < 64 * CPL; idx += 256) {
        const int64_t col = (int64_t)blockIdx.x * 64 * CPL + idx;
        if (col >= cols) continue;
        float vs[4], vq[4];
#pragma unroll
        for (int w = 0; w < 4; w++) vs[w] = part[0][w][idx], vq[w] = part[1][w][idx];
        const float rs = tree_upto<4>(vs, n_waves), rq = tree_upto<4>(vq, n_waves);
        if (n_blocks == 1) {
            if (out_sum) out_sum[col] = rs;
            if (out_sq) out_sq[col] = rq;
        } else {
            ws[(col + (int64_t)blk * cols) * 2] = rs;
            ws[(col + (int64_t)blk * cols) * 2 + 1] = rq;
        }
    }
}

// ---- column axis, one pass ----------------------------------------------------
// For up to 256 leaves per column (rows <= 8192) one workgroup owns a strip
// of 4 * CPL adjacent columns over every row, so no workspace and no second
// kernel are needed.  A lane covers 16 bytes of a row (CPL columns); the 4
// lanes of a quad cover the strip, and quad k of wave w folds the LPQ leaves
// starting at leaf LPQ (16 w + k), each in row order with its 32 rows loaded at
// once (one 64-byte row segment per quad per load instruction); a quad's two
// leaves are its node of tree level 1.  The tree then runs as shuffles at
// lane distances 4, 8, 16, 32 and through LDS over the wave nodes.  LPQ = 2
// for bf16 (8 columns per lane: 512 threads, a leaf's rows fit in registers),
// 1 for fp32 (1024 threads).  The two strips that share a 128-byte line are
// handed to workgroups on one XCD (workgroup b runs on XCD b % 8), so one L2
// fetches the line for both.
template <typename T, bool FUSED>
struct ColFull {
    static constexpr int CPL = 16 / (int)sizeof(T);
    static constexpr int SW = 4 * CPL;              // strip width in columns
    static constexpr int LPQ = CPL == 8 ? 2 : 1;    // leaves per quad
    static constexpr int NW = 16 / LPQ;             // waves: 16 * LPQ * NW = 256 leaves
    static constexpr int NT = 64 * NW;
};

template <typename T, int CPL, bool FUSED>
__device__ __forceinline__ void fold_leaf_rows(const T* base, int64_t ldx, int n, int64_t col0, int64_t cols,
                                               float* s, float* q)
{
    if (n == kLeaf && col0 + CPL <= cols) {
        // the leaf's 32 row pieces stay packed (16 bytes each) until folded
        u32x4 raw[kLeaf];
#pragma unroll
        for (int i = 0; i < kLeaf; i++) raw[i] = *(const u32x4*)(base + i * ldx);
        auto elem = [&](int i, int c) {
            if constexpr (std::is_same<T, float>::value) return __uint_as_float(raw[i][c]);
            else return bf16_lane(raw[i], c);
        };
#pragma unroll
        for (int c = 0; c < CPL; c++) {
            s[c] = elem(0, c);
            q[c] = s[c] * s[c];
        }
#pragma unroll
        for (int i = 1; i < kLeaf; i++)
#pragma unroll
            for (int c = 0; c < CPL; c++) fold_step<FUSED>(elem(i, c), s[c], q[c]);
    } else {
        // a short leaf or the ragged right edge, element by element
        for (int i = 0; i < n; i++) {
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                const float xe = (col0 + c < cols) ? load_elem<T>(base + i * ldx + c) : 0.0f;
                if (i == 0) {
                    s[c] = xe;
                    q[c] = xe * xe;
                } else {
                    fold_step<FUSED>(xe, s[c], q[c]);
                }
            }
        }
    }
}

template <typename T, bool FUSED>
__global__ __launch_bounds__((ColFull<T, FUSED>::NT))
__attribute__((amdgpu_waves_per_eu(ColFull<T, FUSED>::NW / 4, ColFull<T, FUSED>::NW / 4))) void reduce_col_full_kernel(
    const T* __restrict__ X, int64_t ldx, int64_t rows, int64_t cols, float* __restrict__ out_sum,
    float* __restrict__ out_sq)
{
    typedef ColFull<T, FUSED> P;
    constexpr int CPL = P::CPL, SW = P::SW, LPQ = P::LPQ, NW = P::NW;
    __shared__ float part[2][NW][SW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // strip of this workgroup: XCD x gets one contiguous run of strips
    const int n_strips = (int)((cols + SW - 1) / SW);
    const int b = blockIdx.x;
    const int qq = n_strips / 8, rr = n_strips % 8, x = b % 8, j = b / 8;
    const int strip = x * qq + (x < rr ? x : rr) + j;
    const int64_t col0 = (int64_t)strip * SW + (lane & 3) * CPL;
    const int slot = wave * 16 + (lane >> 2);
    const int n_leaf = (int)((rows + kLeaf - 1) / kLeaf);

    float s[CPL], q[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) s[c] = 0.0f, q[c] = 0.0f;
#pragma unroll
    for (int l = 0; l < LPQ; l++) {
        const int leaf = slot * LPQ + l;
        if (leaf < n_leaf) {
            const int64_t r0 = (int64_t)leaf * kLeaf;
            const int n = (int)((rows - r0) < kLeaf ? (rows - r0) : kLeaf);
            float ls[CPL], lq[CPL];
            fold_leaf_rows<T, CPL, FUSED>(X + r0 * ldx + col0, ldx, n, col0, cols, ls, lq);
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                if (l == 0) {
                    s[c] = ls[c];
                    q[c] = lq[c];
                } else {  // tree level 1 inside the quad: (leaf 2k) + (leaf 2k+1)
                    s[c] = s[c] + ls[c];
                    q[c] = q[c] + lq[c];
                }
            }
        }
    }
    // quad-node distances 1, 2, 4, 8 inside the wave (the right node is 4d
    // lanes up); a node exists when its first leaf does
#pragma unroll
    for (int d = 1; d <= 8; d <<= 1) {
        const bool take = (slot & (2 * d - 1)) == 0 && (slot + d) * LPQ < n_leaf;
#pragma unroll
        for (int c = 0; c < CPL; c++) {
            const float os = __shfl_down(s[c], 4 * d, 64);
            const float oq = __shfl_down(q[c], 4 * d, 64);
            if (take) {
                s[c] = s[c] + os;
                q[c] = q[c] + oq;
            }
        }
    }
    if (lane < 4) {
#pragma unroll
        for (int c = 0; c < CPL; c++) {
            part[0][wave][lane * CPL + c] = s[c];
            part[1][wave][lane * CPL + c] = q[c];
        }
    }
    __syncthreads();
    // the wave nodes: node w starts at leaf 16 LPQ w
    if (threadIdx.x < SW) {
        const int c = threadIdx.x;
        const int64_t col = (int64_t)strip * SW + c;
        float vs[NW], vq[NW];
#pragma unroll
        for (int w = 0; w < NW; w++) vs[w] = part[0][w][c], vq[w] = part[1][w][c];
#pragma unroll
        for (int d = 1; d < NW; d <<= 1)
#pragma unroll
            for (int w = 0; w + d < NW; w += 2 * d)
                if (16 * LPQ * (w + d) < n_leaf) {
                    vs[w] = vs[w] + vs[w + d];
                    vq[w] = vq[w] + vq[w + d];
                }
        if (col < cols) {
            if (out_sum) out_sum[col] = vs[0];
            if (out_sq) out_sq[col] = vq[0];
        }
    }
}

// ---- free-order twins (bench only) --------------------------------------------
// Row: coalesced strided lanes (lane l sums elements l*4.., every 1024th
// float4 of the row), a count-down butterfly, an LDS sum over the waves.
template <typename T>
__global__ __launch_bounds__(256) void free_row_kernel(const T* __restrict__ X, int64_t ldx, int64_t cols,
                                                       float* __restrict__ out_sum, float* __restrict__ out_sq)
{
    __shared__ float red[2][4];
    const int64_t row = blockIdx.x;
    const T* xr = X + row * ldx;
    float s = 0.0f, q = 0.0f;
    for (int64_t e = (int64_t)threadIdx.x * 4; e < cols; e += 1024) {
        if (e + 4 <= cols && std::is_same<T, float>::value) {
            const u32x4 v = *(const u32x4*)((const float*)xr + e);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const float x = __uint_as_float(v[j]);
                s += x;
                q = __builtin_fmaf(x, x, q);
            }
        } else {
            for (int64_t j = e; j < e + 4 && j < cols; j++) {
                const float x = load_elem<T>(xr + j);
                s += x;
                q = __builtin_fmaf(x, x, q);
            }
        }
    }
    for (int d = 32; d >= 1; d >>= 1) {
        s += __shfl_xor(s, d, 64);
        q += __shfl_xor(q, d, 64);
    }
    if ((threadIdx.x & 63) == 0) red[0][threadIdx.x >> 6] = s, red[1][threadIdx.x >> 6] = q;
    __syncthreads();
    if (threadIdx.x == 0) {
        if (out_sum) out_sum[row] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
        if (out_sq) out_sq[row] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    }
}

// Column: a grid sized by the CU count; each thread sums a strip of rows of
// one column pair and adds it into the zeroed output with atomics.
template <typename T>
__global__ __launch_bounds__(256) void free_col_kernel(const T* __restrict__ X, int64_t ldx, int64_t rows,
                                                       int64_t cols, int64_t rows_per, float* __restrict__ out_sum,
                                                       float* __restrict__ out_sq)
{
    const int64_t col = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 2;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per;
    if (col >= cols) return;
    float s0 = 0.0f, s1 = 0.0f, q0 = 0.0f, q1 = 0.0f;
    const int64_t r1 = (r0 + rows_per) < rows ? (r0 + rows_per) : rows;
    for (int64_t r = r0; r < r1; r++) {
        const float x0 = load_elem<T>(X + r * ldx + col);
        const float x1 = (col + 1 < cols) ? load_elem<T>(X + r * ldx + col + 1) : 0.0f;
        s0 += x0, s1 += x1;
        q0 = __builtin_fmaf(x0, x0, q0);
        q1 = __builtin_fmaf(x1, x1, q1);
    }
    if (out_sum) {
        atomicAdd(out_sum + col, s0);
        if (col + 1 < cols) atomicAdd(out_sum + col + 1, s1);
    }
    if (out_sq) {
        atomicAdd(out_sq + col, q0);
        if (col + 1 < cols) atomicAdd(out_sq + col + 1, q1);
    }
}

}  // namespace reduce_impl

using namespace reduce_impl;

int64_t reduce_row_blocks(int64_t cols) { return ((cols + kLeaf - 1) / kLeaf + 255) / 256; }

int64_t reduce_col_blocks(int64_t rows, int lpw) { return ((rows + kLeaf - 1) / kLeaf + lpw - 1) / lpw; }

hipError_t launch_reduce(const ReducePlan& p, int64_t rows, int64_t cols, const void* X, int64_t ldx,
                         float* out_sum, float* out_sq, float* ws, hipStream_t stream)
{
    if (p.axis == BG_AXIS_ROW) {
        const int nb = (int)reduce_row_blocks(cols);
        dim3 grid((unsigned)rows, (unsigned)nb), block(256);
#define BG_ROW(T, F)                                                                                          \
    hipLaunchKernelGGL((reduce_row_kernel<T, F>), grid, block, 0, stream, (const T*)X, ldx, cols, out_sum, out_sq, \
                       ws, nb)
        if (p.bf16) {
            if (p.fused) BG_ROW(uint16_t, true);
            else BG_ROW(uint16_t, false);
        } else {
            if (p.fused) BG_ROW(float, true);
            else BG_ROW(float, false);
        }
#undef BG_ROW
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || nb == 1) return e;
        return launch_blocks(ws, rows, nb, (int64_t)nb, (int64_t)1, out_sum, out_sq, stream);
    }
    if (p.col_full) {
        const int sw = p.bf16 ? ColFull<uint16_t, true>::SW : ColFull<float, true>::SW;
        const int nt = p.bf16 ? ColFull<uint16_t, true>::NT : ColFull<float, true>::NT;
        dim3 grid((unsigned)((cols + sw - 1) / sw)), block(nt);
        if (p.bf16) {
            if (p.fused)
                hipLaunchKernelGGL((reduce_col_full_kernel<uint16_t, true>), grid, block, 0, stream, (const uint16_t*)X,
                                   ldx, rows, cols, out_sum, out_sq);
            else
                hipLaunchKernelGGL((reduce_col_full_kernel<uint16_t, false>), grid, block, 0, stream, (const uint16_t*)X,
                                   ldx, rows, cols, out_sum, out_sq);
        } else {
            if (p.fused)
                hipLaunchKernelGGL((reduce_col_full_kernel<float, true>), grid, block, 0, stream, (const float*)X, ldx,
                                   rows, cols, out_sum, out_sq);
            else
                hipLaunchKernelGGL((reduce_col_full_kernel<float, false>), grid, block, 0, stream, (const float*)X, ldx,
                                   rows, cols, out_sum, out_sq);
        }
        return hipGetLastError();
    }
    const int cpl = p.bf16 ? p.cols_per_lane : 4;
    const int lpw = p.leaves_per_wg;
    const int nb = (int)reduce_col_blocks(rows, lpw);
    dim3 grid((unsigned)((cols + 64 * cpl - 1) / (64 * cpl)), (unsigned)nb), block(256);
    bool done = false;
#define BG_COL(T, C, L, F)                                                                                       \
    if (!done && cpl == C && lpw == 4 * L && p.fused == F) {                                                     \
        hipLaunchKernelGGL((reduce_col_kernel<T, C, L, F>), grid, block, 0, stream, (const T*)X, ldx, rows, cols, ws, \
                           out_sum, out_sq, nb);                                                                 \
        done = true;                                                                                             \
    }
#define BG_COL_L(T, C, F) BG_COL(T, C, 1, F) BG_COL(T, C, 2, F) BG_COL(T, C, 4, F) BG_COL(T, C, 8, F)
    if (p.bf16) {
        BG_COL_L(uint16_t, 4, true) BG_COL_L(uint16_t, 4, false) BG_COL_L(uint16_t, 8, true) BG_COL_L(uint16_t, 8, false)
    } else {
        BG_COL_L(float, 4, true) BG_COL_L(float, 4, false)
    }
#undef BG_COL_L
#undef BG_COL
    if (!done) return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || nb == 1) return e;
    return launch_col_blocks(ws, cols, nb, out_sum, out_sq, stream);
}

hipError_t launch_reduce_free(int axis, bool bf16, int64_t rows, int64_t cols, const void* X, int64_t ldx,
                              float* out_sum, float* out_sq, int n_cu, hipStream_t stream)
{
    if (axis == BG_AXIS_ROW) {
        if (bf16)
            hipLaunchKernelGGL(free_row_kernel<uint16_t>, dim3((unsigned)rows), dim3(256), 0, stream,
                               (const uint16_t*)X, ldx, cols, out_sum, out_sq);
        else
            hipLaunchKernelGGL(free_row_kernel<float>, dim3((unsigned)rows), dim3(256), 0, stream, (const float*)X,
                               ldx, cols, out_sum, out_sq);
        return hipGetLastError();
    }
    // zero the outputs (a fill kernel, so the sequence can be graph-captured),
    // then one strip per CU-sized slot
    if (out_sum) {
        hipError_t e = launch_zero_rows(out_sum, 1, cols, cols, stream);
        if (e != hipSuccess) return e;
    }
    if (out_sq) {
        hipError_t e = launch_zero_rows(out_sq, 1, cols, cols, stream);
        if (e != hipSuccess) return e;
    }
    const int64_t col_wgs = (cols + 511) / 512;
    int64_t strips = (4 * (int64_t)n_cu + col_wgs - 1) / col_wgs;
    if (strips < 1) strips = 1;
    const int64_t rows_per = (rows + strips - 1) / strips;
    dim3 grid((unsigned)col_wgs, (unsigned)((rows + rows_per - 1) / rows_per)), block(256);
    if (bf16)
        hipLaunchKernelGGL(free_col_kernel<uint16_t>, grid, block, 0, stream, (const uint16_t*)X, ldx, rows, cols,
                           rows_per, out_sum, out_sq);
    else
        hipLaunchKernelGGL(free_col_kernel<float>, grid, block, 0, stream, (const float*)X, ldx, rows, cols, rows_per,
                           out_sum, out_sq);
    return hipGetLastError();
}

hipError_t launch_leaf_tree(const float* ws_sum, const float* ws_sq, int64_t n_out, int n_leaf, float* out_sum,
                            float* out_sq, hipStream_t stream)
{
    dim3 grid((unsigned)((n_out + 63) / 64)), block(1024);
    hipLaunchKernelGGL(leaf_tree_kernel, grid, block, 0, stream, ws_sum, ws_sq, n_out, n_leaf, out_sum, out_sq);
    return hipGetLastError();
}

}  // namespace bg
