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
// row.  Each wave copies its 64 leaves with coalesced global_load_lds loads
// (16 B per lane, consecutive lanes on consecutive addresses) into LDS; each
// lane then reads its own leaf back, rotating its chunk order by its lane
// index so that the 16-byte reads of a wave spread over the banks.
// Column axis: lanes map to adjacent columns (coalesced rows), each lane
// folds its columns' leaves row by row; a workgroup covers an aligned run of
// leaves with its waves, combined through LDS.
#include <type_traits>

#include "bg_internal.h"

namespace bg {

namespace reduce_impl {

constexpr int kLeaf = 32;

__device__ __forceinline__ void lds_copy16(const void* src, u32x4* lds_dst)
{
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

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

// Balanced tree over up to 8 workgroup-level nodes held in LDS (node i
// covering 2^level_base leaves each), n_valid of them present.
__device__ __forceinline__ float small_tree(float* v, int n)
{
    while (n > 1) {
        int w = 0;
        for (int i = 0; i + 1 < n; i += 2) v[w++] = v[i] + v[i + 1];
        if (n & 1) v[w++] = v[n - 1];
        n = w;
    }
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
// One workgroup: row `row`, leaf block `blk` (256 leaves).  fp32 input with a
// full block on the fast path (direct copies to LDS); anything else (bf16, a
// short block, an unaligned row) folds straight from global memory.
template <typename T, bool FUSED>
__global__ __launch_bounds__(256) void reduce_row_kernel(const T* __restrict__ X, int64_t ldx, int64_t cols,
                                                         float* __restrict__ out_sum, float* __restrict__ out_sq,
                                                         float* __restrict__ ws, int n_blocks)
{
    __shared__ u32x4 stage[4 * 64 * 8];  // 4 waves x 64 leaves x 128 B (fp32)
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
    const bool full = std::is_same<T, float>::value && (leaf0 + 256) * kLeaf <= cols;
    if (full) {
        // coalesced copy of this wave's 64 leaves (8 KB) into LDS
        const float* src = (const float*)xr + (leaf0 + wave * 64) * kLeaf;
#pragma unroll
        for (int c = 0; c < 8; c++) lds_copy16(src + (c * 64 + lane) * 4, &stage[(wave * 8 + c) * 64]);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float x[kLeaf];
        const u32x4* mine = &stage[(wave * 64 + lane) * 8];
#pragma unroll
        for (int c = 0; c < 8; c++) {
            const int cc = (c + lane) & 7;  // rotated chunk order: spreads the banks
            const u32x4 v = mine[cc];
#pragma unroll
            for (int j = 0; j < 4; j++) x[cc * 4 + j] = __uint_as_float(v[j]);
        }
        fold_leaf<FUSED>(x, kLeaf, s, q);
    } else if (my_leaf < n_valid) {
        const int64_t e0 = (leaf0 + my_leaf) * kLeaf;
        const int n = (int)((cols - e0) < kLeaf ? (cols - e0) : kLeaf);
        float x[kLeaf];
        for (int i = 0; i < n; i++) x[i] = load_elem<T>(xr + e0 + i);
        fold_leaf<FUSED>(x, n, s, q);
    }

    // wave level: this wave's nodes are leaves [64 wave, 64 wave + 64)
    const int wave_valid = n_valid - wave * 64;
    s = wave_tree(s, lane, wave_valid);
    q = wave_tree(q, lane, wave_valid);
    if (lane == 0) {
        roots[0][wave] = s;
        roots[1][wave] = q;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int n_waves = (n_valid + 63) / 64;
        float vs[4], vq[4];
        for (int w = 0; w < n_waves; w++) vs[w] = roots[0][w], vq[w] = roots[1][w];
        const float rs = small_tree(vs, n_waves), rq = small_tree(vq, n_waves);
        if (n_blocks == 1) {
            if (out_sum) out_sum[row] = rs;
            if (out_sq) out_sq[row] = rq;
        } else {
            ws[(row * n_blocks + blk) * 2] = rs;
            ws[(row * n_blocks + blk) * 2 + 1] = rq;
        }
    }
}

// Upper tree levels over the block roots of one output.
__global__ __launch_bounds__(256) void reduce_blocks_kernel(const float* __restrict__ ws, int64_t n_out,
                                                            int n_blocks, int64_t stride_out, int64_t stride_blk,
                                                            float* __restrict__ out_sum, float* __restrict__ out_sq)
{
    const int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (o >= n_out) return;
    float vs[64], vq[64];  // n_blocks <= 64 (checked by the host)
    for (int b = 0; b < n_blocks; b++) {
        vs[b] = ws[(o * stride_out + b * stride_blk) * 2];
        vq[b] = ws[(o * stride_out + b * stride_blk) * 2 + 1];
    }
    const float rs = small_tree(vs, n_blocks), rq = small_tree(vq, n_blocks);
    if (out_sum) out_sum[o] = rs;
    if (out_sq) out_sq[o] = rq;
}

// ---- column axis ------------------------------------------------------------
// A workgroup covers CPL * 64 adjacent columns and LPW leaves (LPW * 32 rows)
// starting at leaf block `blk`; wave w folds leaves [w LPW/4, (w+1) LPW/4)
// of that run, one after the other, pairing them as they complete.
template <typename T, int CPL, int LPW, bool FUSED>
__global__ __launch_bounds__(256) void reduce_col_kernel(const T* __restrict__ X, int64_t ldx, int64_t rows,
                                                         int64_t cols, float* __restrict__ ws,
                                                         float* __restrict__ out_sum, float* __restrict__ out_sq,
                                                         int n_blocks)
{
    constexpr int LPWAVE = LPW / 4;  // leaves per wave (a power of two)
    __shared__ float part[2][4][64 * CPL];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t col0 = (int64_t)blockIdx.x * 64 * CPL + lane * CPL;
    const int blk = blockIdx.y;
    const int64_t n_leaf = (rows + kLeaf - 1) / kLeaf;
    const int64_t wleaf0 = (int64_t)blk * LPW + wave * LPWAVE;  // this wave's first leaf

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
        auto fold_rows = [&](int nr) {
        for (int i = 0; i < nr; i++) {
            const T* p = X + (r0 + i) * ldx + col0;
            float x[CPL];
            if (col0 + CPL <= cols) {
                if constexpr (std::is_same<T, float>::value) {
                    const u32x4 v = *(const u32x4*)p;  // CPL == 4 for fp32
#pragma unroll
                    for (int c = 0; c < CPL; c++) x[c] = __uint_as_float(v[c]);
                } else {
                    if constexpr (CPL == 8) {
                        const u32x4 v = *(const u32x4*)p;
#pragma unroll
                        for (int c = 0; c < 4; c++) {
                            x[2 * c] = __uint_as_float(v[c] << 16);
                            x[2 * c + 1] = __uint_as_float(v[c] & 0xffff0000u);
                        }
                    } else {
                        const uint2 v = *(const uint2*)p;
                        x[0] = __uint_as_float(v.x << 16);
                        x[1] = __uint_as_float(v.x & 0xffff0000u);
                        x[2] = __uint_as_float(v.y << 16);
                        x[3] = __uint_as_float(v.y & 0xffff0000u);
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < CPL; c++) x[c] = (col0 + c < cols) ? load_elem<T>(p + c) : 0.0f;
            }
#pragma unroll
            for (int c = 0; c < CPL; c++) {
                if (i == 0) {
                    s[c] = x[c];
                    q[c] = x[c] * x[c];
                } else {
                    s[c] = s[c] + x[c];
                    if constexpr (FUSED) q[c] = __builtin_fmaf(x[c], x[c], q[c]);
                    else {
                        const float xx = x[c] * x[c];
                        q[c] = q[c] + xx;
                    }
                }
            }
        }
        };
        if (n == kLeaf) {
#pragma unroll
            for (int h = 0; h < 1; h++) fold_rows(kLeaf);
        } else {
            fold_rows(n);
        }
#pragma unroll
        for (int c = 0; c < CPL; c++) ls[l][c] = s[c], lq[l][c] = q[c];
    }
    // this wave's leaves -> one node (balanced, neighbours first, odd carried)
    float ws_[CPL], wq_[CPL];
#pragma unroll
    for (int c = 0; c < CPL; c++) {
        float vs[LPWAVE], vq[LPWAVE];
        for (int l = 0; l < n_mine; l++) vs[l] = ls[l][c], vq[l] = lq[l][c];
        ws_[c] = n_mine ? small_tree(vs, n_mine) : 0.0f;
        wq_[c] = n_mine ? small_tree(vq, n_mine) : 0.0f;
    }
#pragma unroll
    for (int c = 0; c < CPL; c++) {
        part[0][wave][lane * CPL + c] = ws_[c];
        part[1][wave][lane * CPL + c] = wq_[c];
    }
    __syncthreads();
    // the workgroup's waves -> one node; waves with no leaf do not exist
    const int64_t blk_leaf0 = (int64_t)blk * LPW;
    const int n_waves = (int)(((n_leaf - blk_leaf0) + LPWAVE - 1) / LPWAVE < 4 ? ((n_leaf - blk_leaf0) + LPWAVE - 1) / LPWAVE : 4);
    for (int idx = threadIdx.x; idx < 64 * CPL; idx += 256) {
        const int64_t col = (int64_t)blockIdx.x * 64 * CPL + idx;
        if (col >= cols) continue;
        float vs[4], vq[4];
        for (int w = 0; w < n_waves; w++) vs[w] = part[0][w][idx], vq[w] = part[1][w][idx];
        const float rs = small_tree(vs, n_waves), rq = small_tree(vq, n_waves);
        if (n_blocks == 1) {
            if (out_sum) out_sum[col] = rs;
            if (out_sq) out_sq[col] = rq;
        } else {
            ws[(col + (int64_t)blk * cols) * 2] = rs;
            ws[(col + (int64_t)blk * cols) * 2 + 1] = rq;
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
        dim3 g2((unsigned)((rows + 255) / 256));
        hipLaunchKernelGGL(reduce_blocks_kernel, g2, dim3(256), 0, stream, ws, rows, nb, (int64_t)nb, (int64_t)1,
                           out_sum, out_sq);
        return hipGetLastError();
    }
    const int cpl = p.bf16 ? p.cols_per_lane : 4;
    const int lpw = p.leaves_per_wg;
    const int nb = (int)reduce_col_blocks(rows, lpw);
    dim3 grid((unsigned)((cols + 64 * cpl - 1) / (64 * cpl)), (unsigned)nb), block(256);
    bool done = false;
#define BG_COL(T, C, L, F)                                                                                       \
    if (!done && cpl == C && lpw == L && p.fused == F) {                                                         \
        hipLaunchKernelGGL((reduce_col_kernel<T, C, L, F>), grid, block, 0, stream, (const T*)X, ldx, rows, cols, ws, \
                           out_sum, out_sq, nb);                                                                 \
        done = true;                                                                                             \
    }
#define BG_COL_L(T, C, F) BG_COL(T, C, 4, F) BG_COL(T, C, 8, F) BG_COL(T, C, 16, F) BG_COL(T, C, 32, F)
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
    dim3 g2((unsigned)((cols + 255) / 256));
    hipLaunchKernelGGL(reduce_blocks_kernel, g2, dim3(256), 0, stream, ws, cols, nb, (int64_t)1, cols, out_sum,
                       out_sq);
    return hipGetLastError();
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
    // zero the outputs with a kernel-free memset, then one strip per CU-sized slot
    if (out_sum) {
        hipError_t e = hipMemsetAsync(out_sum, 0, cols * sizeof(float), stream);
        if (e != hipSuccess) return e;
    }
    if (out_sq) {
        hipError_t e = hipMemsetAsync(out_sq, 0, cols * sizeof(float), stream);
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

}  // namespace bg
