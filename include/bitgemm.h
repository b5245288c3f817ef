/*
 * bitgemm.h -- C ABI of libbitgemm: GEMMs and reductions whose floating-point
 * reduction order is fixed by an explicit descriptor, for AMD Instinct MI355X
 * (gfx950).  Two calls with equal order fields return equal bits, whatever the
 * batch size, the tile schedule or the number of compute units.
 *
 * Passages each entry point follows (cited by page title and section):
 *   [T]  "Taming Bitwise Behavior in GPU Kernels with Tensor Core: Black-Box
 *        Reconstruction, Compiler Enforcement, and Static Verification"
 *        (arXiv 2609.11356).  3.1 dependence tree of a reduction; 3.2.1 one
 *        rounding per matrix instruction; 3.2.2 the GEMM descriptor fields
 *        (instruction_k, k_loop_step, span, k_cuts, partial_dtype,
 *        merge_dtype); 4 the frozen descriptor (identical records, identical
 *        bits) and the black-box +L/-L/r instruments; 5.1 the
 *        count-up, neighbours-first lane tree; appendix E (a descriptor fixes
 *        the arithmetic, not the schedule; host cost of a descriptor path).
 *   [E]  "GPU Arithmetic Emulator" README, "Tensor Core Matmul" (block-FMA
 *        model of one instruction; returning the raw fp32 accumulator).
 *   [W]  "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
 *        Quantization Scales and the Limits of Tolerance-Based Conformance",
 *        section II (Y = (A W^T) s_a s_w, exact INT32 accumulation,
 *        power-of-two commutation).
 *   [G]  "GPU Mechanism" page, forced-algorithm section: a request the device
 *        cannot honour is refused, never silently replaced by another order.
 *
 * Conventions for every entry point:
 *   - Memory: every tensor and workspace pointer is a DEVICE pointer owned by
 *     the caller.  The library allocates no device memory on any call path.
 *     Descriptors are plain structs owned by the caller, passed by const
 *     pointer and only read during the call.
 *   - Execution: work is enqueued on `stream` (NULL = the default stream) and
 *     the call returns without synchronising.  Device faults surface at the
 *     caller's next synchronisation.
 *   - Errors: invalid arguments are reported synchronously by the status code,
 *     with a message from bg_last_error() (thread-local).  A launch failure is
 *     BG_E_HIP.  No C++ exception crosses the ABI.  On any non-BG_OK status no
 *     work has been enqueued.
 *   - Refusal: a descriptor the library cannot realise exactly (an unsupported
 *     field value, a profile measured on another device) is refused with
 *     BG_E_UNSUPPORTED / BG_E_PROFILE; another order is never substituted [G].
 *   - Size: each call is one launch (or a short fixed sequence), and a
 *     dispatch counts each grid dimension's work-items in 32 bits; a shape
 *     whose grid would pass that is refused with BG_E_UNSUPPORTED.  Limits per
 *     call are stated with it where they bind before memory runs out.
 *   - Alignment: tensor pointers 16-byte aligned; leading dimensions a
 *     multiple of 8 elements (bf16, fp32) or 16 (int8); else BG_E_ALIGN.
 *   - Thread safety: calls are reentrant.  Calls that share a workspace must be
 *     ordered by the caller (same stream, or events).
 */
#ifndef BITGEMM_H
#define BITGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t; /* the HIP runtime's stream handle */

#define BG_ABI_VERSION 2
#define BG_MAX_SPLIT 64

typedef enum {
    BG_OK = 0,
    BG_E_INVALID = 1,     /* malformed descriptor or arguments            */
    BG_E_UNSUPPORTED = 2, /* well-formed, but the library cannot realise it */
    BG_E_WORKSPACE = 3,   /* workspace missing or too small               */
    BG_E_ALIGN = 4,       /* pointer or leading dimension misaligned      */
    BG_E_ARCH = 5,        /* the current device is not gfx950             */
    BG_E_PROFILE = 6,     /* descriptor's MFMA profile is not the library's */
    BG_E_HIP = 7          /* a HIP runtime call failed                    */
} bg_status;

typedef enum { BG_FP32 = 0, BG_BF16 = 1, BG_INT8 = 2, BG_INT32 = 3 } bg_dtype;

/* The matrix instruction, named one by one ([T] 3.2.1): it is fixed per
 * descriptor and used for every M. */
typedef enum {
    BG_MFMA_F32_32X32X16_BF16 = 0, /* instruction_k = 16 */
    BG_MFMA_F32_16X16X32_BF16 = 1, /* instruction_k = 32 */
    BG_MFMA_I32_32X32X32_I8 = 2,   /* instruction_k = 32 */
    BG_MFMA_I32_16X16X64_I8 = 3    /* instruction_k = 64 */
} bg_mfma;

typedef enum { BG_ACC_IN_MFMA = 0, BG_ACC_SEPARATE_ADD = 1 } bg_acc_update;   /* [T] use_fast_accum */
typedef enum { BG_K_ASCENDING = 0 } bg_k_order;
typedef enum { BG_SHORT_TURN_LAST = 0, BG_SHORT_TURN_FIRST = 1 } bg_short_turn; /* [T] k_loop_step */
typedef enum { BG_SLOTS_CONTIGUOUS = 0, BG_SLOTS_STRIDED = 1 } bg_slot_layout;  /* [T] layout */
typedef enum { BG_CUT_UNIT_REMAINDER_LAST = 0, BG_CUT_EXPLICIT = 1 } bg_cut_rule;
typedef enum { BG_COMBINE_BALANCED = 0, BG_COMBINE_SEQUENTIAL = 1 } bg_combine;
typedef enum { BG_ODD_CARRY_LAST = 0 } bg_odd_rule;
typedef enum { BG_ROUND_AFTER_COMBINE_RNE = 0 } bg_rounding_point;
typedef enum { BG_EPI_NONE = 0, BG_EPI_W8A8_POW2 = 1 } bg_epilogue;

/* Speed knobs.  They are NOT part of the order: any value returns the same
 * bits ([T] 3.2.2: BLOCK_M/N/K are speed knobs; appendix E).  bm..waves_n all
 * 0 = let the library choose the tile and load path for the shape; a
 * combination that is not compiled in is BG_E_UNSUPPORTED. */
typedef struct {
    int32_t bm, bn, bk;       /* output tile and k-tile                    */
    int32_t waves_m, waves_n; /* wave grid inside a workgroup              */
    int32_t load_path;        /* 0: global -> VGPR -> LDS; 1: global -> LDS;
                                 2: global -> LDS, multi-stage pipeline (k
                                 tiles of 32 or 64; 32x32x16 instruction
                                 only; 64-deep tiles in two stages address
                                 their copies by 32-bit offsets and need
                                 (bm - 1) x lda and (bn - 1) x ldb below
                                 2^31 elements)                            */
    int32_t group_m;          /* tile rows per group of the workgroup walk
                                 (0 = 8; for path 2, the height that makes
                                 each XCD's concurrent tiles fetch the
                                 fewest A and B rows)                      */
    int32_t stages;           /* k tiles held in LDS by path 2 (0 = the
                                 tile's default); for W8A8 on path 2, two
                                 or three stages take 128-byte k tiles
                                 (two stages address their copies by
                                 32-bit offsets), four or more 64-byte
                                 ones                                      */
    int32_t last_bm, last_bn; /* path 2 with split_k > 1: the last split
                                 (the cut rule's remainder, the deepest)
                                 takes this tile in the same launch; all
                                 five last_* 0 = the same tile as the other
                                 splits.  Needs bm..waves_n set; the pair
                                 must be compiled in and have the same
                                 number of waves                           */
    int32_t last_waves_m, last_waves_n;
    int32_t last_stages;
} bg_gemm_schedule;

/* GEMM descriptor ([T] 3.2.2 and 4).  Every field before `sched` is an order
 * field and is hashed by bg_desc_signature(). */
typedef struct {
    uint32_t version;        /* 1                                            */
    uint32_t a_type, b_type; /* BG_BF16 (bg_gemm_bf16) or BG_INT8 (W8A8)     */
    uint32_t acc_type;       /* BG_FP32 or BG_INT32                          */
    uint32_t out_type;       /* BG_FP32 or BG_BF16                           */
    uint32_t mfma;           /* bg_mfma                                      */
    uint32_t acc_update;     /* BG_ACC_IN_MFMA                               */
    uint32_t k_order;        /* BG_K_ASCENDING                               */
    uint32_t short_turn;     /* BG_SHORT_TURN_LAST: a short last turn is
                                zero-padded                                  */
    uint32_t k_slot_layout;  /* BG_SLOTS_CONTIGUOUS                          */
    uint32_t split_k;        /* S, 1..BG_MAX_SPLIT                           */
    uint32_t cut_rule;       /* bg_cut_rule                                  */
    uint32_t cut_unit;       /* unit of the span rule (256)                  */
    int64_t cuts[BG_MAX_SPLIT + 1]; /* explicit cut points (cut_rule EXPLICIT):
                                cuts[0] = 0 < cuts[1] < ... < cuts[S] = K,
                                each a multiple of 8                          */
    uint32_t partial_type;   /* BG_FP32                                      */
    uint32_t merge_type;     /* BG_FP32                                      */
    uint32_t combine;        /* BG_COMBINE_BALANCED                          */
    uint32_t odd_rule;       /* BG_ODD_CARRY_LAST                            */
    uint32_t rounding_point; /* BG_ROUND_AFTER_COMBINE_RNE                   */
    uint32_t epilogue;       /* BG_EPI_NONE or BG_EPI_W8A8_POW2              */
    uint64_t mfma_profile_hash; /* must equal bg_profile_hash()              */
    bg_gemm_schedule sched;  /* not hashed                                   */
} bg_gemm_desc;

typedef enum { BG_RED_SUM = 1, BG_RED_SUMSQ = 2, BG_RED_SUM_AND_SUMSQ = 3 } bg_reduce_op;
typedef enum { BG_AXIS_ROW = 0, BG_AXIS_COL = 1 } bg_axis;
typedef enum { BG_LEAF_SEQUENTIAL_NO_SEED = 0 } bg_leaf_order;
typedef enum { BG_SQ_FUSED = 0, BG_SQ_UNFUSED = 1 } bg_sq_fma;
typedef enum { BG_TREE_BALANCED = 0 } bg_tree;

typedef struct {
    int32_t leaves_per_wg;  /* column axis: leaves one workgroup folds: 4, 8, 16
                               or 32 (0: 4 for bf16 and 8 for fp32 input,
                               raised until <= 64 block roots remain);
                               256: one pass, a workgroup per narrow column
                               strip over every row (rows <= 8192)          */
    int32_t cols_per_wg;    /* column axis: columns one workgroup covers: 256,
                               or 512 for bf16 (0: 256)                        */
    int32_t reserved0, reserved1;
} bg_reduce_schedule;

/* Reduction descriptor ([T] 3.1 and 5.1): leaves of leaf_len consecutive
 * elements of the reduced axis folded in index order with no +0 seed, then a
 * balanced binary tree over the leaf index, neighbours first, an odd element
 * carried up.  The tree never depends on the number of compute units. */
typedef struct {
    uint32_t version;    /* 1                                  */
    uint32_t in_type;    /* BG_FP32 or BG_BF16                 */
    uint32_t acc_type;   /* BG_FP32                            */
    uint32_t op;         /* bg_reduce_op                       */
    uint32_t axis;       /* bg_axis                            */
    uint32_t leaf_len;   /* 32                                 */
    uint32_t leaf_order; /* BG_LEAF_SEQUENTIAL_NO_SEED         */
    uint32_t sq_fma;     /* BG_SQ_FUSED: q = fma(x, x, q)      */
    uint32_t tree;       /* BG_TREE_BALANCED                   */
    uint32_t odd_rule;   /* BG_ODD_CARRY_LAST                  */
    uint32_t out_type;   /* BG_FP32                            */
    bg_reduce_schedule sched; /* not hashed                    */
} bg_reduce_desc;

/* ---- housekeeping ------------------------------------------------------ */
int bg_abi_version(void);
const char* bg_status_str(bg_status s);
const char* bg_last_error(void); /* message of this thread's last failure */

/* Hash of the MFMA arithmetic profile this library was built against: the
 * black-box measurement of how a gfx950 instruction sums its products ([T] 4,
 * [E]).  Descriptors carry it; a mismatch is BG_E_PROFILE. */
uint64_t bg_profile_hash(void);

/* Fill a descriptor with the defaults: bf16 x bf16 -> fp32 acc, bf16 out,
 * 32x32x16 instruction, S = 1, balanced combine, the library's profile hash. */
bg_status bg_desc_default_gemm(bg_gemm_desc* d);
bg_status bg_desc_default_reduce(bg_reduce_desc* d);

/* Descriptors as JSON text: the frozen record of [T] 4 in the form it is
 * stored and handed between tools (the oracle reads the same text).
 * Document: {"gemm": {...}, "reduce": {...}}, either member optional; the
 * keys are the struct field names (the schedule as a "schedule" object),
 * enum values by name ("bf16", "F32_32X32X16_BF16", "EXPLICIT", "row",
 * "fused", ...), integers as plain JSON integers, mfma_profile_hash as a
 * string "0x" + 16 hex digits, and "cuts" an array of split_k + 1 points.
 * bg_desc_from_json: g and/or r (either may be NULL, not both) are set to
 *   the defaults of bg_desc_default_gemm / bg_desc_default_reduce with the
 *   document's fields applied.  A malformed document, an unknown key, a value
 *   of the wrong type or name, or a cut table of another length is
 *   BG_E_INVALID and leaves g and r untouched.  It reads the record only;
 *   whether the library can realise it is decided by the call that uses it.
 * bg_desc_to_json: writes every field of g and/or r (NULL skips it) as one
 *   NUL-terminated document into buf (host memory, cap bytes); *len (if not
 *   NULL) gets the text's length without the NUL.  cap too small (or buf
 *   NULL) is BG_E_INVALID with *len set.  A field holding a value that has
 *   no name is BG_E_INVALID.  Reading the text back gives equal order
 *   fields, schedule and signature. */
bg_status bg_desc_from_json(const char* json, bg_gemm_desc* g, bg_reduce_desc* r);
bg_status bg_desc_to_json(const bg_gemm_desc* g, const bg_reduce_desc* r, char* buf, size_t cap, size_t* len);

/* 128-bit signature over the order fields only (FNV-1a, two lanes).  Equal
 * signatures mean equal arithmetic ([T] 4). */
bg_status bg_desc_signature(const bg_gemm_desc* d, uint64_t sig[2]);
bg_status bg_reduce_desc_signature(const bg_reduce_desc* d, uint64_t sig[2]);

/* Cut points the descriptor gives for K: cuts[0..split_k], host memory
 * provided by the caller.  Unit rule: span = floor(K / (unit*S)) * unit for
 * every split but the last, which takes the remainder ([T] 3.2.2 span);
 * an empty span is BG_E_INVALID. */
bg_status bg_gemm_split_cuts(const bg_gemm_desc* d, int64_t K, int64_t* cuts);

/* Workspace bytes a GEMM call needs: S * M * N * 4 for S > 1 (the fp32 split
 * partials), else 0. */
bg_status bg_gemm_workspace_bytes(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K,
                                  size_t* bytes);

/* ---- the hot path -------------------------------------------------------- */

/* The tiles bg_gemm_bf16 would launch for this descriptor and shape (host
 * only: no device, no memory read): the descriptor's schedule, or the
 * library's choice (a speed knob, [T] 3.2.2; for split_k > 1 the last split
 * may take its own tile, last_*).  lda = ldb = K and ldc = N are assumed.
 * M or N of 0 is BG_E_INVALID (nothing would launch); any descriptor or size
 * bg_gemm_bf16 refuses is refused with the same status. */
bg_status bg_gemm_bf16_plan(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K, bg_gemm_schedule* out);

/* C = A * B^T in bf16 with fp32 accumulation, order fixed by d ([T] 3.2):
 *   for each output (m, n) and split s: acc = +0; for the blocks of
 *   instruction_k consecutive k in ascending order inside [cut_s, cut_s+1)
 *   (a short last block zero-padded): acc = MFMA(acc, block).  Each split's
 *   acc is an fp32 partial (workspace [S][M][N]); the partials are combined by
 *   a balanced tree, neighbours first, with no atomics; the result is rounded
 *   once to out_type (fp32: stored as is; bf16: round to nearest even).
 * A: bf16 [M][lda], row-major, K contiguous (activations).
 * B: bf16 [N][ldb], row-major, K contiguous (weights; C = A B^T).
 * C: fp32 or bf16 [M][ldc] per d->out_type.
 * ws: device workspace of at least bg_gemm_workspace_bytes() (NULL if 0).
 * M, N >= 0, K >= 1; M or N = 0 enqueues nothing. */
bg_status bg_gemm_bf16(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K,
                       const void* A, int64_t lda, const void* B, int64_t ldb,
                       void* C, int64_t ldc, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* bg_gemm_bf16 for callers that cannot allocate device memory or hand in a
 * workspace (code under stream or graph capture, tight serving loops,
 * harnesses that forbid allocation): the same descriptor, arguments, order,
 * kernels and bits as bg_gemm_bf16, with the split-K partials kept in a
 * static scratch inside the library instead of a caller workspace.
 * The scratch is 64 MiB per GPU (S * M * N * 4 bytes at most; e.g. split-K 16
 * at 256 x 2560 takes 42 MB), allocated with the library's code object on
 * each GPU it runs on and held until the process ends; a call that needs
 * more is refused with BG_E_WORKSPACE before anything is enqueued.  The call
 * itself allocates nothing.  Every call on one GPU shares that GPU's scratch:
 * calls that can overlap in time on one GPU (different streams without
 * ordering) race on it and must be ordered by the caller.  S = 1 uses no
 * scratch. */
bg_status bg_gemm_bf16_noalloc(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K,
                               const void* A, int64_t lda, const void* B, int64_t ldb,
                               void* C, int64_t ldc, hipStream_t stream);

/* W8A8 with power-of-two weight scales ([W] section II):
 *   acc[m][n] = sum_k A[m][k] * W[n][k] in exact int32 (order-free: |acc| <=
 *   K * 127^2 must stay below 2^31, so K <= 133,144);
 *   Y[m][n] = bf16_rne( fp32( fp32_rne(acc) * w_scale[n] ) * a_scale[m] ).
 * A: int8 [M][lda]; W: int8 [N][ldw]; a_scale: fp32 [M]; w_scale: fp32 [N]
 * (powers of two -- a precondition, not checked on the hot path).
 * Y: bf16 [M][ldy].  acc_out: optional int32 [M][ld_acc] raw accumulators
 * (NULL to skip).  d->epilogue must be BG_EPI_W8A8_POW2, d->split_k 1. */
bg_status bg_gemm_w8a8_pow2(const bg_gemm_desc* d, int64_t M, int64_t N, int64_t K,
                            const int8_t* A, int64_t lda, const int8_t* W, int64_t ldw,
                            const float* a_scale, const float* w_scale,
                            void* Y, int64_t ldy, int32_t* acc_out, int64_t ld_acc,
                            hipStream_t stream);

/* ---- GEMM with fused reductions of C -------------------------------------- */

/* C = A * B^T exactly as bg_gemm_bf16 (split_k must be 1; the 32x32x16
 * instruction), plus a fixed-order reduction of the fp32 C values -- the
 * accumulators before any rounding to out_type -- along one axis, in the
 * tree bg_reduce_tree applies ([T] 3.1 and 5.1; [T]'s evaluation of
 * performance cost, Figures 5(b) and 6, fuses such epilogues, a GEMM's
 * column sum among them): rd->axis COL gives one output per
 * column n over the rows of C (a bias-gradient style column sum), ROW one per
 * row m over its columns (norm statistics); leaves of 32 consecutive elements
 * folded in index order with no seed, then a balanced tree over the leaves.
 * The result equals bg_reduce_tree(rd) applied to the fp32 C of the same
 * GEMM.  rd->in_type must be FP32; the reduced axis holds at most 1024 leaves;
 * K must be a multiple of 8 (BG_E_UNSUPPORTED otherwise, as bg_gemm_bf16
 * requires of every cut point).
 * out_sum / out_sumsq: fp32 [N] (COL) or [M] (ROW), NULL where rd->op leaves
 * them out.  ws: at least bg_gemm_bf16_reduce_workspace_bytes() bytes, 4-byte
 * aligned (one fp32 node per leaf and output).  M or N = 0 enqueues nothing
 * and writes no output. */
bg_status bg_gemm_bf16_reduce_workspace_bytes(const bg_gemm_desc* d, const bg_reduce_desc* rd, int64_t M,
                                              int64_t N, int64_t K, size_t* bytes);
bg_status bg_gemm_bf16_reduce(const bg_gemm_desc* d, const bg_reduce_desc* rd, int64_t M, int64_t N, int64_t K,
                              const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                              float* out_sum, float* out_sumsq, void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- Ozaki-scheme GEMM ----------------------------------------------------- */

/* C = A * B^T by the Ozaki scheme ("GPU Mechanism", the exact-GEMM
 * paragraph and intervention (a)): every row of A and of B is scaled by 2^-e
 * (e the frexp exponent of its largest magnitude; 0 for a zero row) and cut
 * into four signed pieces of 7 bits, r = 128 r, q = trunc(r), r = r - q; the
 * 16 piece products are exact int32 dot products (int8 MFMA: an integer sum
 * comes out the same whatever order its terms arrive in, so tiling and CU
 * count cannot reach the result); per output the scaled products acc_st 2^(-7 (s + t + 2)) are added
 * in fp64 in the fixed order s + t = 6 .. 0, s ascending within a level,
 * scaled by 2^(eA + eB) and rounded once to out_type (nearest even).  The
 * accuracy is fp32-class: slices keep 28 bits below each row's largest
 * element.  Inputs must be finite.
 * A: [M][lda], B: [N][ldb] of in_type (BG_FP32 or BG_BF16), K contiguous;
 * C: [M][ldc] of out_type.  ws: at least bg_gemm_ozaki_workspace_bytes(),
 * 16-byte aligned (the slices and exponents; the products are recombined
 * where the int8 GEMM produces them and never written out).
 * M, N < 2^24 and M * N < 2^32; K rounded up to 16 at most 133,144. */
bg_status bg_gemm_ozaki_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes);
bg_status bg_gemm_ozaki(int64_t M, int64_t N, int64_t K, uint32_t in_type, const void* A, int64_t lda,
                        const void* B, int64_t ldb, uint32_t out_type, void* C, int64_t ldc, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/* ---- int8 quantisation on either side of W8A8 ----------------------------- */

/* Per-token int8 quantisation of activations (the input of bg_gemm_w8a8_pow2;
 * the pages run W8A8 on int8 activations without printing this step, and this
 * is the plainest per-token absmax reading):
 *   a_scale[m] = fp32(max_k |X[m][k]|) / 127, rounded once (1 for a row of
 *   zeros); Q[m][k] = clamp(rint(X[m][k] / a_scale[m]), -127, 127), the
 *   division rounded once, rint taking ties to even, a NaN quotient giving 0.
 *   The maximum is exact, so the result does not depend on any order.
 * X: fp32 [M][ldx] (device, caller-owned); Q: int8 [M][ldq]; a_scale: fp32 [M].
 * Inputs are expected finite (an infinite element makes its row's scale
 * infinite and its codes 0).  M, K >= 0, M < 2^24; X and Q may be NULL when
 * K = 0 (every scale is then 1); X 4-byte aligned (16-byte X rows with
 * K % 4 == 0 take the vector path).  Errors come back synchronously with
 * nothing enqueued. */
bg_status bg_quantize_act_int8(int64_t M, int64_t K, const float* X, int64_t ldx, int8_t* Q, int64_t ldq,
                               float* a_scale, hipStream_t stream);

/* Requantisation of int8 weights to power-of-two scales ("Deterministic LLM
 * Inference ... Power-of-Two INT8 Quantization Scales", section V: the
 * int8 weights themselves are recomputed for the power-of-two scale;
 * changing the scale alone would not do), per output row n:
 *   s2 = 2^e, e = round(log2 w_scale[n]) for BG_POW2_NEAREST (nearest in
 *   ratio; decided exactly, a tie cannot occur) or e = ceil(log2 w_scale[n])
 *   for BG_POW2_CEIL (never shrinks the scale, so nothing clips);
 *   W2[n][k] = clamp(rint(fp32(W[n][k] * w_scale[n]) / s2), -127, 127).
 *   A row whose scale is not a positive finite number is copied unchanged.
 * W, W2: int8 [N][ldw] / [N][ldw2] (may not overlap); w_scale, w_scale2:
 * fp32 [N].  N, K >= 0, N < 2^25 - 1 (W and W2 may be NULL when K = 0).  The
 * outputs feed bg_gemm_w8a8_pow2. */
enum { BG_POW2_NEAREST = 0, BG_POW2_CEIL = 1 };
bg_status bg_requantize_weights_pow2(int64_t N, int64_t K, const int8_t* W, int64_t ldw, const float* w_scale,
                                     uint32_t mode, int8_t* W2, int64_t ldw2, float* w_scale2,
                                     hipStream_t stream);

/* Workspace bytes bg_reduce_tree needs (column axis: one fp32 partial per
 * column per workgroup row-block). */
bg_status bg_reduce_workspace_bytes(const bg_reduce_desc* d, int64_t rows, int64_t cols,
                                    size_t* bytes);

/* Fixed-order sum and/or sum of squares ([T] 3.1, 5.1):
 *   axis ROW: out[r] over X[r][0..cols); axis COL: out[c] over X[0..rows)[c].
 *   leaf j folds elements [32j, 32j+32) of the reduced axis in index order
 *   (s = x0; s = s + xi; q = x0*x0; q = fma(xi, xi, q)), then a balanced tree
 *   over the leaf index.  Both outputs come from one read of X.
 * X: fp32 or bf16 [rows][ldx] per d->in_type.  out_sum / out_sumsq: fp32
 * [rows] (ROW) or [cols] (COL); NULL to skip (per d->op).  Axis ROW takes
 * rows < 2^24 (a workgroup per row). */
bg_status bg_reduce_tree(const bg_reduce_desc* d, int64_t rows, int64_t cols,
                         const void* X, int64_t ldx, float* out_sum, float* out_sumsq,
                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ---- free-order twins (bench only; no bitwise contract) -------------------
 * The same arithmetic with the order left free, as the denominator of the
 * cost of holding the order: split-K chosen from the CU count and combined
 * with fp32 atomics into a zeroed C (fp32 out only); reductions with
 * coalesced strided lanes, a count-down butterfly and, for columns, atomics.
 * split_k <= 0 lets the library pick. */
bg_status bg_bench_gemm_bf16_free(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                  const void* B, int64_t ldb, float* C, int64_t ldc,
                                  int32_t split_k, hipStream_t stream);
/* Another free-order twin of the same product ([T] 3.2.1: the chain of
 * roundings across instructions is what survives as the order; 3.2.2: a
 * strided deal of the axis over accumulators is another order): each output
 * carries two interleaved fp32 chains, even 16-deep k-steps into one and odd
 * ones into the other, added once after the walk -- the reassociation an
 * implementation free to reorder may use to hide the instruction's latency.
 * The 128x128 tile with 64-deep k tiles in a ring of four (the same main loop
 * as that tile's order-fixed kernel, selectable through the descriptor's
 * schedule), fp32 C [M][ldc].  Same argument rules as bg_gemm_bf16 (K a
 * multiple of 8; 127 x lda x 2 + 128 and 127 x ldb x 2 + 128 below 2^32). */
bg_status bg_bench_gemm_bf16_two_chains(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                        const void* B, int64_t ldb, float* C, int64_t ldc, hipStream_t stream);
/* W8A8 with the epilogue's order left free: the same tile, main loop and
 * exact int32 sums as bg_gemm_w8a8_pow2, then y = bf16(fp32(acc) *
 * (a_scale[m] * w_scale[n])) -- the two scales combined first, as an
 * implementation free to reorder would.  With power-of-two w_scale this gives
 * the same bits ([W] section II: power-of-two commutation); it is the
 * denominator of what holding the epilogue's order costs. */
bg_status bg_bench_gemm_w8a8_free(int64_t M, int64_t N, int64_t K, const int8_t* A, int64_t lda,
                                  const int8_t* W, int64_t ldw, const float* a_scale, const float* w_scale,
                                  void* Y, int64_t ldy, hipStream_t stream);
bg_status bg_bench_reduce_free(uint32_t axis, uint32_t in_type, int64_t rows, int64_t cols,
                               const void* X, int64_t ldx, float* out_sum, float* out_sumsq,
                               hipStream_t stream);

/* ---- black-box instrument ----------------------------------------------
 * Runs exactly one matrix instruction per wavefront on caller-crafted tiles,
 * so that how the instruction sums its products can be reconstructed from
 * outside ([T] 4; [E]).  For case i (one wave):
 *   bf16 32x32x16: A [32][16], B [32][16] (B holds rows n, i.e. B^T),
 *                  C, D fp32 [32][32];  D = MFMA(C, A, B^T)
 *   bf16 16x16x32: A [16][32], B [16][32], C, D [16][16]
 *   i8   32x32x32: A [32][32], B [32][32] int8, C, D int32 [32][32]
 *   i8   16x16x64: A [16][64], B [16][64] int8, C, D int32 [16][16]
 * All row-major and packed case after case.  Element k of row m of A and row
 * n of B is the instruction's k-th product slot, in the same lane/register
 * placement the GEMM kernels use.  n_cases < 2^26. */
bg_status bg_probe_mfma(uint32_t mfma, int64_t n_cases, const void* A, const void* B,
                        const void* C, void* D, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* BITGEMM_H */
