/*
 * bg_oracle.h -- CPU oracle for the fixed-order GEMM and reductions.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the bench may load this library.  It shares no code,
 * header, table or helper with the GPU library; the only thing both sides
 * agree on is the descriptor (a JSON document) and the seeded input bytes.
 *
 * Everything here is written to be read against the pages, not to be fast:
 *   - "Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv
 *     2609.11356), section 3.1 (dependence tree of a reduction), section
 *     3.2.1 (tensor-core semantics: one rounding per instruction over an exact
 *     sum), section 3.2.2 (instruction_k, k_loop_step, split-K span / k_cuts /
 *     partial_dtype / merge_dtype, "a second kernel sums the parts"), section 4
 *     (the +L/-L/r walks), section 5.1 (count-up, neighbours-first tree).
 *   - "GPU Arithmetic Emulator" README, section "Tensor Core Matmul": block
 *     FMA with products kept exact, a max exponent over products and
 *     accumulator, an alignment window of 2+23+neab bits with truncation, an
 *     integer sum, truncation to fp32; CoFDA (chained groups) vs FDA.
 *   - "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
 *     Quantization Scales ...", section II (Y = (A W^T) s_a s_w with exact
 *     INT32 accumulation; power-of-two commutation).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -fopenmp -shared
 * (the emulator page's rule: keep the host compiler from fusing mul+add).
 */
#ifndef BG_ORACLE_H
#define BG_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- one matrix instruction, as a model ---------------------------------
 * The pages give two readings of how one tensor-core instruction sums its
 * products (they disagree even for NVIDIA, and neither measures gfx950):
 *   family E ("Taming", 3.2.1): acc <- round(acc + sum_j a_j b_j), the sum
 *            exact, one rounding.  Here: frac_bits = OR_EXACT, acc in window.
 *   family B (emulator README): products exact; e_max over the products and
 *            the accumulator; every term cut to a window whose lowest kept bit
 *            sits frac_bits below e_max (2+23+neab window -> frac_bits =
 *            23+neab); integer sum; truncation to fp32.
 * Both are instances of one parameterised step: the products of a group are
 * aligned to their largest exponent, cut to a window (or not), summed exactly
 * together with the accumulator, and rounded once.  Groups of `group`
 * products are chained in slot order (CoFDA when group < instruction_k).
 * The step is also written with the accumulator joining in a second stage
 * (OR_ACC_TWO_STAGE), because "Taming" section 4 is explicit that where the
 * roundings fall inside an instruction is a black box to be read off from
 * outside, and its two-instrument method applied to gfx950 finds such a
 * second stage.  Which member describes a given instruction is settled by
 * that experiment; this file only evaluates a member faithfully. */
#define OR_EXACT (-1)

enum { OR_ROUND_RNE = 0, OR_ROUND_RZ = 1 };
enum { OR_EXP_RAW = 0,   /* product exponent = ea + eb, significand in [1,4) */
       OR_EXP_NORM = 1 }; /* exponent of the leading set bit of the exact value */
enum { OR_TRUNC_TOWARD_ZERO = 0, /* drop the bits of the magnitude (sign-magnitude) */
       OR_TRUNC_FLOOR = 1 };     /* drop the bits of the two's complement (toward -inf) */
enum { OR_ACC_IN_WINDOW = 0, /* the acc is one more term of the group's aligned sum:
                                e_max over products and acc, every term cut to the
                                window, one rounding (both families of the pages) */
       OR_ACC_SEPARATE = 1,  /* the group's products summed and rounded alone, then
                                one fp32 add into the acc (two roundings)          */
       OR_ACC_TWO_STAGE = 2 }; /* the products cut to their own window (e_max over
                                the products only) and the acc cut to the same
                                lowest bit, all summed exactly; then the sum is
                                normalised, every bit more than acc_frac_bits below
                                its leading bit dropped, and rounded once          */

typedef struct {
    int32_t group;         /* products per fused group, 1..instruction_k       */
    int32_t frac_bits;     /* window bits below the reference exponent, or
                              OR_EXACT for no cut                              */
    int32_t exp_mode;      /* OR_EXP_RAW | OR_EXP_NORM                         */
    int32_t acc_mode;      /* OR_ACC_IN_WINDOW | OR_ACC_SEPARATE | OR_ACC_TWO_STAGE */
    int32_t acc_frac_bits; /* OR_ACC_TWO_STAGE: bits kept below the sum's
                              leading bit before the rounding                 */
    int32_t round;         /* OR_ROUND_RNE | OR_ROUND_RZ for a group's result  */
    int32_t trunc;         /* how a product's bits below the window are dropped */
    int32_t acc_trunc;     /* the same for the accumulator                     */
    int32_t sum_trunc;     /* OR_ACC_TWO_STAGE: the same for that last cut     */
    int32_t slot_order[64]; /* slot_order[i] = the k of the i-th product fed
                               to the adder; identity when slot_order[0] < 0   */
} or_mfma_model;

/* ---- scalar primitives --------------------------------------------------- */
uint16_t or_bf16_rne(float x);              /* fp32 -> bf16, ties to even     */
float    or_f32_from_bf16(uint16_t h);      /* exact                          */
float    or_f32_from_i32(int32_t v);        /* RNE (C conversion, default FE) */
void     or_bf16_rne_n(const float* x, uint16_t* y, int64_t n);
float    or_f32_round_sum(int n, const int32_t* sign, const uint64_t* mag,
                          const int32_t* exp2, int round_mode);
            /* exact sum of n terms (-1)^sign * mag * 2^exp2, rounded once */

/* One instruction: acc' = MFMA(acc, a[0..k), b[0..k)) under model m.
 * a and b are bf16 bit patterns indexed by k. */
float or_mfma_bf16(const or_mfma_model* m, float acc,
                   const uint16_t* a, const uint16_t* b, int k);

/* n independent instructions: out[i] = MFMA(acc[i], a[i][0..k), b[i][0..k)) */
void or_mfma_bf16_batch(const or_mfma_model* m, int64_t n, int k, const float* acc,
                        const uint16_t* a, const uint16_t* b, float* out, int32_t n_threads);

/* ---- GEMM walk ----------------------------------------------------------
 * C = A * B^T with A [M][lda] and B [N][ldb] bf16 (K contiguous in both).
 * For every (m, n) and split s: acc = +0; for k-blocks of instr_k in
 * ascending k inside [cuts[s], cuts[s+1]) (the last block zero-padded):
 * acc = MFMA(acc, block).  Partials combined by `combine`, then rounded once
 * to out_type. */
enum { OR_COMBINE_BALANCED = 0, OR_COMBINE_SEQUENTIAL = 1 };
enum { OR_OUT_F32 = 0, OR_OUT_BF16 = 1 };

typedef struct {
    or_mfma_model model;
    int32_t instr_k;
    int32_t n_split;
    int64_t cuts[65];   /* n_split + 1 cut points, cuts[0] = 0, cuts[S] = K */
    int32_t combine;
    int32_t out_type;
} or_gemm_desc;

/* Cut rule "unit 256, remainder last": span = floor(K / (unit*S)) * unit for
 * every split but the last; the last gets the rest.  Returns 0, or -1 when a
 * span would be empty. */
int or_split_cuts(int64_t K, int S, int64_t unit, int64_t* cuts);

/* Balanced tree, neighbours first, an odd last element carried up unchanged.
 * Overwrites v. */
float or_tree_balanced(float* v, int n);

/* one output element; partials (length n_split) may be NULL */
float or_gemm_elem(const or_gemm_desc* d, int64_t K,
                   const uint16_t* arow, const uint16_t* brow, float* partials);

/* Full output.  C is float [M][ldc] or uint16 [M][ldc] per out_type. */
void or_gemm_bf16(const or_gemm_desc* d, int64_t M, int64_t N, int64_t K,
                  const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                  void* C, int64_t ldc, int32_t n_threads);

/* Selected outputs (m_idx[i], n_idx[i]); out is float or uint16 per out_type. */
void or_gemm_bf16_points(const or_gemm_desc* d, int64_t K,
                         const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                         int64_t n_pts, const int64_t* m_idx, const int64_t* n_idx,
                         void* out, int32_t n_threads);

/* ---- W8A8 with power-of-two weight scales ------------------------------
 * acc = sum_k A[m][k] * W[n][k] exactly (plain definition, int64, must fit
 * int32); y = bf16_rne( fp32( fp32(acc) * w_scale[n] ) * a_scale[m] ).
 * Returns 0, or -1 if some accumulator left the int32 range. */
int or_w8a8_pow2(int64_t M, int64_t N, int64_t K,
                 const int8_t* A, int64_t lda, const int8_t* W, int64_t ldw,
                 const float* a_scale, const float* w_scale,
                 uint16_t* Y, int64_t ldy, int32_t* acc_out, int64_t ld_acc,
                 int32_t n_threads);

/* ---- int8 quantisation on either side of W8A8 ---------------------------
 * Activations, per token (per row): scale = fp32(max |x|) / 127, one
 * rounding (an all-zero row takes scale 1); q = clamp(rint(x / scale),
 * -127, 127), the division rounded once and rint taking ties to even; a NaN
 * quotient (from a non-finite input) gives 0.  The pages run W8A8 on int8
 * activations without printing this step; this is the plainest reading of
 * per-token absmax quantisation.
 *
 * Weights, per output row ("Deterministic LLM Inference ... Power-of-Two
 * INT8 Quantization Scales", section V: requantise the int8 weights under the
 * constrained scale rather than only rewriting the scale): s2 = 2^e with
 * e = round(log2 s) (mode 0, nearest in ratio, decided exactly by s^2 against
 * 2^(2e-1)) or e = ceil(log2 s) (mode 1, never shrinks the scale); each
 * weight becomes clamp(rint(fp32(q * s) / s2), -127, 127): the product
 * rounded once, the division by a power of two exact.  A row whose scale is
 * not a positive finite number is copied unchanged. */
void or_quantize_rows_int8(int64_t M, int64_t K, const float* X, int64_t ldx,
                           int8_t* Q, int64_t ldq, float* scale, int32_t n_threads);
enum { OR_POW2_NEAREST = 0, OR_POW2_CEIL = 1 };
float or_pow2_scale(float s, int mode);
void or_requantize_pow2(int64_t N, int64_t K, const int8_t* W, int64_t ldw, const float* w_scale,
                        int mode, int8_t* W2, int64_t ldw2, float* w_scale2, int32_t n_threads);

/* ---- Ozaki-scheme GEMM ("GPU Mechanism", exact GEMM by error-free
 * transformation, intervention (a)) -------------------------------------
 * C = A B^T with A [M][K], B [N][K] (fp32, or bf16 bits when in_bf16).  Each
 * row x of A and of B: e = the frexp exponent of max |x| (0 for a zero row);
 * r = x * 2^-e in [-1, 1); for s = 0..3: r = r * 128, q_s = trunc(r) (an int8
 * in [-127, 127]), r = r - q_s.  For each output and each slice pair (s, t):
 * acc_st = sum_k qA_s[m][k] * qB_t[n][k] exactly (an integer: no order).  The
 * value sum over pairs of acc_st * 2^(-7 (s + t + 2)) is added in fp64 in the
 * fixed order s + t = 6, 5, ..., 0 (least significant first), s ascending
 * within a level; it is scaled by 2^(eA_m + eB_n) and rounded once to the
 * output (fp32, or bf16 when out_bf16; round to nearest even).  Returns -1
 * if a slice product left the int32 range (K > 133,144). */
int or_ozaki_gemm(int64_t M, int64_t N, int64_t K, int in_bf16, const void* A, int64_t lda, const void* B,
                  int64_t ldb, int out_bf16, void* C, int64_t ldc, int32_t n_threads);
/* The slicing of one row (K elements): q [4][K] int8, returns e. */
int or_ozaki_slice_row(int64_t K, int in_bf16, const void* x, int8_t* q);
/* double -> bf16 bits, one rounding (nearest even). */
uint16_t or_bf16_from_f64(double v);

/* ---- fixed-order reductions ---------------------------------------------
 * out[i] = balanced tree over leaf sums; a leaf is leaf_len consecutive
 * elements of the reduced axis folded in index order with no +0 seed
 * (sum: s = x0, s = s + xi; sumsq: s = x0*x0, s = fma(xi, xi, s) when
 * sq_fused, else s = s + xi*xi with two roundings).  The last leaf may be
 * short.  axis 0: reduce along a row (one output per row); axis 1: reduce
 * down a column (one output per column). */
enum { OR_IN_F32 = 0, OR_IN_BF16 = 1 };
enum { OR_AXIS_ROW = 0, OR_AXIS_COL = 1 };
void or_reduce(int in_type, int axis, int64_t rows, int64_t cols,
               const void* X, int64_t ldx, int32_t leaf_len, int32_t sq_fused,
               float* out_sum, float* out_sumsq, int32_t n_threads);

int or_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
