"""CPU oracle for the fixed-order GEMM, split-K combine, W8A8 and reductions.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the bench's
CPU-baseline leg, never by the library.  It shares no code with the GPU path;
the two agree only on the descriptor JSON and the seeded input bytes.

The arithmetic lives in bg_oracle.c (plain C, one exact wide accumulator);
this module only marshals numpy arrays and descriptor dicts into it.  Each
function names the passage it follows:

* "Taming Bitwise Behavior in GPU Kernels with Tensor Core" (arXiv 2609.11356):
  section 3.1 (dependence tree, in-register fold in index order, n-1 work),
  3.2.1 (one rounding per instruction over an exact sum), 3.2.2 (instruction_k,
  k_loop_step, split-K span/k_cuts, partial_dtype/merge_dtype, second-kernel
  merge), 4 (the +L/-L/r walks), 5.1 (count-up neighbours-first tree).
* "GPU Arithmetic Emulator" README, "Tensor Core Matmul" (block FMA window
  model, CoFDA vs FDA).
* "Deterministic LLM Inference Across GPU Kernels: Power-of-Two INT8
  Quantization Scales" section II (exact INT32 accumulation; epilogue order).
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

OR_EXACT = -1
ROUND = {"rne": 0, "rz": 1}
EXP_MODE = {"raw": 0, "norm": 1}
TRUNC = {"toward_zero": 0, "floor": 1}
ACC_MODE = {"in_window": 0, "separate": 1, "two_stage": 2}
COMBINE = {"BALANCED_NEIGHBOURS_FIRST": 0, "SEQUENTIAL": 1}
OUT = {"fp32": 0, "bf16": 1}
INSTR_K = {"F32_32X32X16_BF16": 16, "F32_16X16X32_BF16": 32}


class _Model(C.Structure):
    _fields_ = [("group", C.c_int32), ("frac_bits", C.c_int32),
                ("exp_mode", C.c_int32), ("acc_mode", C.c_int32),
                ("acc_frac_bits", C.c_int32), ("round", C.c_int32),
                ("trunc", C.c_int32), ("acc_trunc", C.c_int32), ("sum_trunc", C.c_int32),
                ("slot_order", C.c_int32 * 64)]


class _GemmDesc(C.Structure):
    _fields_ = [("model", _Model), ("instr_k", C.c_int32), ("n_split", C.c_int32),
                ("cuts", C.c_int64 * 65), ("combine", C.c_int32),
                ("out_type", C.c_int32)]


_lib = None


def lib():
    """Load liboracle.so, building it first only if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        L.or_bf16_rne.restype = C.c_uint16
        L.or_bf16_rne.argtypes = [C.c_float]
        L.or_bf16_rne_n.argtypes = [P, P, C.c_int64]
        L.or_f32_from_i32.restype = C.c_float
        L.or_f32_from_i32.argtypes = [C.c_int32]
        L.or_f32_round_sum.restype = C.c_float
        L.or_f32_round_sum.argtypes = [C.c_int, P, P, P, C.c_int]
        L.or_mfma_bf16.restype = C.c_float
        L.or_mfma_bf16.argtypes = [P, C.c_float, P, P, C.c_int]
        L.or_mfma_bf16_batch.argtypes = [P, C.c_int64, C.c_int, P, P, P, P, C.c_int32]
        L.or_split_cuts.restype = C.c_int
        L.or_split_cuts.argtypes = [C.c_int64, C.c_int, C.c_int64, P]
        L.or_tree_balanced.restype = C.c_float
        L.or_tree_balanced.argtypes = [P, C.c_int]
        L.or_gemm_elem.restype = C.c_float
        L.or_gemm_elem.argtypes = [P, C.c_int64, P, P, P]
        L.or_gemm_bf16.argtypes = [P, C.c_int64, C.c_int64, C.c_int64, P, C.c_int64,
                                   P, C.c_int64, P, C.c_int64, C.c_int32]
        L.or_gemm_bf16_points.argtypes = [P, C.c_int64, P, C.c_int64, P, C.c_int64,
                                          C.c_int64, P, P, P, C.c_int32]
        L.or_w8a8_pow2.restype = C.c_int
        L.or_w8a8_pow2.argtypes = [C.c_int64, C.c_int64, C.c_int64, P, C.c_int64, P,
                                   C.c_int64, P, P, P, C.c_int64, P, C.c_int64, C.c_int32]
        L.or_reduce.argtypes = [C.c_int, C.c_int, C.c_int64, C.c_int64, P, C.c_int64,
                                C.c_int32, C.c_int32, P, P, C.c_int32]
        L.or_quantize_rows_int8.argtypes = [C.c_int64, C.c_int64, P, C.c_int64, P, C.c_int64, P, C.c_int32]
        L.or_pow2_scale.restype = C.c_float
        L.or_pow2_scale.argtypes = [C.c_float, C.c_int]
        L.or_requantize_pow2.argtypes = [C.c_int64, C.c_int64, P, C.c_int64, P, C.c_int, P, C.c_int64, P,
                                         C.c_int32]
        L.or_ozaki_gemm.restype = C.c_int
        L.or_ozaki_gemm.argtypes = [C.c_int64, C.c_int64, C.c_int64, C.c_int, P, C.c_int64, P, C.c_int64, C.c_int,
                                    P, C.c_int64, C.c_int32]
        L.or_ozaki_slice_row.restype = C.c_int
        L.or_ozaki_slice_row.argtypes = [C.c_int64, C.c_int, P, P]
        L.or_bf16_from_f64.restype = C.c_uint16
        L.or_bf16_from_f64.argtypes = [C.c_double]
        L.or_abi_version.restype = C.c_int
        _lib = L
    return _lib


def _ptr(a):
    return C.c_void_p(a.ctypes.data) if a is not None else None


def default_threads():
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


# --------------------------------------------------------------------------
# models of one instruction
# --------------------------------------------------------------------------
def model_struct(model):
    """Descriptor dict -> C struct.  Keys: group, frac_bits (None = no cut),
    exp_mode ('raw'|'norm'), acc_mode ('in_window'|'separate'|'two_stage'),
    acc_frac_bits (two_stage), round ('rne'|'rz'), trunc / acc_trunc /
    sum_trunc ('toward_zero'|'floor'; the latter two default to trunc),
    slot_order (None = k order)."""
    m = _Model()
    m.group = int(model["group"])
    fb = model.get("frac_bits")
    m.frac_bits = OR_EXACT if fb is None else int(fb)
    m.exp_mode = EXP_MODE[model.get("exp_mode", "raw")]
    m.acc_mode = ACC_MODE[model.get("acc_mode", "in_window")]
    m.acc_frac_bits = int(model.get("acc_frac_bits") or 0)
    m.round = ROUND[model.get("round", "rne")]
    m.trunc = TRUNC[model.get("trunc", "toward_zero")]
    m.acc_trunc = TRUNC[model.get("acc_trunc", model.get("trunc", "toward_zero"))]
    m.sum_trunc = TRUNC[model.get("sum_trunc", model.get("trunc", "toward_zero"))]
    so = model.get("slot_order")
    if so is None:
        m.slot_order[0] = -1
    else:
        for i, v in enumerate(so):
            m.slot_order[i] = int(v)
    return m


def family_e(instr_k=16):
    """'Taming', section 3.2.1: exact sum of the instruction's products and the
    accumulator, one RNE rounding."""
    return {"group": instr_k, "frac_bits": None, "exp_mode": "raw",
            "acc_mode": "in_window", "round": "rne", "trunc": "toward_zero"}


def family_b(nfma=16, neab=2):
    """Emulator README, 'Tensor Core Matmul': window of 2+23+neab bits below the
    max exponent (so 23+neab fraction bits), truncation, RZ to fp32; groups of
    NFMA products chained (CoFDA when NFMA < instruction_k)."""
    return {"group": nfma, "frac_bits": 23 + neab, "exp_mode": "raw",
            "acc_mode": "in_window", "round": "rz", "trunc": "toward_zero"}


def mfma_bf16(model, acc, a_bits, b_bits):
    """One instruction: acc' = MFMA(acc, a, b) under `model` (bf16 bit arrays)."""
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16)
    m = model_struct(model)
    return float(np.float32(lib().or_mfma_bf16(C.byref(m), C.c_float(acc), _ptr(a), _ptr(b), len(a))))


def mfma_bf16_batch(model, acc, a_bits, b_bits, threads=None):
    """Many independent instructions: acc [n] f32, a/b [n][k] bf16 bits."""
    acc = np.ascontiguousarray(acc, dtype=np.float32)
    a = np.ascontiguousarray(a_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_bits, dtype=np.uint16)
    assert a.shape == b.shape and a.shape[0] == acc.shape[0]
    m = model_struct(model)
    out = np.empty(acc.shape[0], dtype=np.float32)
    lib().or_mfma_bf16_batch(C.byref(m), acc.shape[0], a.shape[1], _ptr(acc), _ptr(a), _ptr(b),
                             _ptr(out), threads or default_threads())
    return out


# --------------------------------------------------------------------------
# scalar helpers
# --------------------------------------------------------------------------
def bf16_rne(x):
    """fp32 -> bf16 bits, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(x.shape, dtype=np.uint16)
    lib().or_bf16_rne_n(_ptr(x), _ptr(y), x.size)
    return y if y.ndim else y[()]


def bf16_to_f32(h):
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_from_i32(v):
    return float(np.float32(lib().or_f32_from_i32(int(v))))


def round_sum(terms, mode="rne"):
    """Exact sum of terms [(sign, mag, exp2)], one rounding to fp32."""
    n = len(terms)
    s = np.array([t[0] for t in terms], dtype=np.int32)
    m = np.array([t[1] for t in terms], dtype=np.uint64)
    e = np.array([t[2] for t in terms], dtype=np.int32)
    return float(np.float32(lib().or_f32_round_sum(n, _ptr(s), _ptr(m), _ptr(e), ROUND[mode])))


def split_cuts(K, S, unit=256):
    """Cut rule: span = floor(K/(unit*S))*unit, remainder to the last split.
    Raises ValueError when a span would be empty."""
    cuts = np.zeros(S + 1, dtype=np.int64)
    if lib().or_split_cuts(int(K), int(S), int(unit), _ptr(cuts)) != 0:
        raise ValueError(f"no split of K={K} into {S} parts of unit {unit}")
    return [int(c) for c in cuts]


def tree_balanced(values):
    """Balanced tree over the values, neighbours first, odd element carried."""
    v = np.array(values, dtype=np.float32)
    return float(np.float32(lib().or_tree_balanced(_ptr(v), len(v))))


# --------------------------------------------------------------------------
# GEMM
# --------------------------------------------------------------------------
def gemm_desc_struct(desc, K):
    """Descriptor dict -> C struct.  desc keys: mfma, mfma_model, split_k,
    cut_rule ('UNIT256_REMAINDER_LAST'|'EXPLICIT'), cuts, cut_unit, combine,
    out_type."""
    d = _GemmDesc()
    d.model = model_struct(desc["mfma_model"])
    d.instr_k = INSTR_K[desc.get("mfma", "F32_32X32X16_BF16")]
    S = int(desc.get("split_k", 1))
    if desc.get("cut_rule", "UNIT256_REMAINDER_LAST") == "EXPLICIT":
        cuts = [int(c) for c in desc["cuts"]]
        if len(cuts) != S + 1 or cuts[0] != 0 or cuts[-1] != K or any(
                cuts[i] >= cuts[i + 1] for i in range(S)):
            raise ValueError(f"bad explicit cuts {cuts} for K={K}, S={S}")
    else:
        cuts = split_cuts(K, S, int(desc.get("cut_unit", 256)))
    d.n_split = S
    for i, c in enumerate(cuts):
        d.cuts[i] = c
    d.combine = COMBINE[desc.get("combine", "BALANCED_NEIGHBOURS_FIRST")]
    d.out_type = OUT[desc.get("out_type", "fp32")]
    return d


def gemm_bf16(desc, A_bits, B_bits, threads=None):
    """C = A B^T, A [M][K], B [N][K] bf16 bits.  Returns float32 [M][N] or
    uint16 (bf16 bits) [M][N] per desc['out_type']."""
    A = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B_bits, dtype=np.uint16)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    d = gemm_desc_struct(desc, K)
    out = np.empty((M, N), dtype=np.uint16 if d.out_type == 1 else np.float32)
    lib().or_gemm_bf16(C.byref(d), M, N, K, _ptr(A), K, _ptr(B), K, _ptr(out), N,
                       threads or default_threads())
    return out


def gemm_bf16_points(desc, A_bits, B_bits, m_idx, n_idx, threads=None):
    """Selected outputs of C = A B^T."""
    A = np.ascontiguousarray(A_bits, dtype=np.uint16)
    B = np.ascontiguousarray(B_bits, dtype=np.uint16)
    K = A.shape[1]
    d = gemm_desc_struct(desc, K)
    mi = np.ascontiguousarray(m_idx, dtype=np.int64)
    ni = np.ascontiguousarray(n_idx, dtype=np.int64)
    assert mi.shape == ni.shape
    assert mi.size == 0 or (mi.min() >= 0 and mi.max() < A.shape[0] and ni.min() >= 0 and ni.max() < B.shape[0])
    out = np.empty(mi.shape, dtype=np.uint16 if d.out_type == 1 else np.float32)
    lib().or_gemm_bf16_points(C.byref(d), K, _ptr(A), K, _ptr(B), K, mi.size, _ptr(mi),
                              _ptr(ni), _ptr(out), threads or default_threads())
    return out


def gemm_partials(desc, a_row_bits, b_row_bits):
    """(final value, per-split partials) for one output element."""
    a = np.ascontiguousarray(a_row_bits, dtype=np.uint16)
    b = np.ascontiguousarray(b_row_bits, dtype=np.uint16)
    d = gemm_desc_struct(desc, a.size)
    p = np.zeros(d.n_split, dtype=np.float32)
    v = lib().or_gemm_elem(C.byref(d), a.size, _ptr(a), _ptr(b), _ptr(p))
    return float(np.float32(v)), p


# --------------------------------------------------------------------------
# W8A8
# --------------------------------------------------------------------------
def w8a8_pow2(A_q, W_q, a_scale, w_scale, threads=None):
    """Y = bf16( fp32( fp32(acc) * w_scale[n] ) * a_scale[m] ), acc exact.
    Returns (Y bf16 bits [M][N], acc int32 [M][N])."""
    A = np.ascontiguousarray(A_q, dtype=np.int8)
    W = np.ascontiguousarray(W_q, dtype=np.int8)
    a_s = np.ascontiguousarray(a_scale, dtype=np.float32)
    w_s = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = A.shape
    N = W.shape[0]
    Y = np.empty((M, N), dtype=np.uint16)
    acc = np.empty((M, N), dtype=np.int32)
    rc = lib().or_w8a8_pow2(M, N, K, _ptr(A), K, _ptr(W), K, _ptr(a_s), _ptr(w_s),
                            _ptr(Y), N, _ptr(acc), N, threads or default_threads())
    if rc != 0:
        raise OverflowError("an int8 accumulator left the int32 range")
    return Y, acc


# --------------------------------------------------------------------------
# int8 quantisation on either side of W8A8
# --------------------------------------------------------------------------
def quantize_rows_int8(X, threads=None):
    """Per-token absmax int8 quantisation of float32 X [M][K].  Returns
    (Q int8 [M][K], scale float32 [M])."""
    X = np.ascontiguousarray(X, dtype=np.float32)
    M, K = X.shape
    Q = np.empty((M, K), dtype=np.int8)
    s = np.empty(M, dtype=np.float32)
    lib().or_quantize_rows_int8(M, K, _ptr(X), K, _ptr(Q), K, _ptr(s), threads or default_threads())
    return Q, s


POW2_MODES = {"nearest": 0, "ceil": 1}


def pow2_scale(s, mode="nearest"):
    """The power-of-two scale that replaces scale s."""
    return float(np.float32(lib().or_pow2_scale(float(np.float32(s)), POW2_MODES[mode])))


def requantize_pow2(W, w_scale, mode="nearest", threads=None):
    """Requantise int8 W [N][K] with scales w_scale [N] to power-of-two
    scales.  Returns (W2 int8 [N][K], s2 float32 [N])."""
    W = np.ascontiguousarray(W, dtype=np.int8)
    s = np.ascontiguousarray(w_scale, dtype=np.float32)
    N, K = W.shape
    W2 = np.empty((N, K), dtype=np.int8)
    s2 = np.empty(N, dtype=np.float32)
    lib().or_requantize_pow2(N, K, _ptr(W), K, _ptr(s), POW2_MODES[mode], _ptr(W2), K, _ptr(s2),
                             threads or default_threads())
    return W2, s2


# --------------------------------------------------------------------------
# Ozaki-scheme GEMM
# --------------------------------------------------------------------------
def ozaki_gemm(A, B, in_type="fp32", out_type="fp32", threads=None):
    """C = A B^T from four signed 7-bit pieces per operand row: the piece
    products are exact integers, summed in fp64 in a set order, rounded once.  A, B: float32
    arrays, or uint16 bf16 bits with in_type='bf16'.  Returns float32 or
    uint16 (bf16 bits)."""
    dt = np.uint16 if in_type == "bf16" else np.float32
    A = np.ascontiguousarray(A, dtype=dt)
    B = np.ascontiguousarray(B, dtype=dt)
    M, K = A.shape
    N = B.shape[0]
    C_out = np.empty((M, N), dtype=np.uint16 if out_type == "bf16" else np.float32)
    rc = lib().or_ozaki_gemm(M, N, K, int(in_type == "bf16"), _ptr(A), K, _ptr(B), K, int(out_type == "bf16"),
                             _ptr(C_out), N, threads or default_threads())
    if rc != 0:
        raise OverflowError("a slice product left the int32 range")
    return C_out


def ozaki_slice_row(x, in_type="fp32"):
    """(q int8 [4][K], e) for one row."""
    dt = np.uint16 if in_type == "bf16" else np.float32
    x = np.ascontiguousarray(x, dtype=dt)
    q = np.empty((4, x.size), dtype=np.int8)
    e = lib().or_ozaki_slice_row(x.size, int(in_type == "bf16"), _ptr(x), _ptr(q))
    return q, e


def bf16_from_f64(v):
    return int(lib().or_bf16_from_f64(float(v)))


# --------------------------------------------------------------------------
# reductions
# --------------------------------------------------------------------------
def reduce(X, axis, leaf_len=32, sq_fused=True, in_type=None, threads=None):
    """Fixed-order sum and sum of squares.  X float32 [rows][cols], or uint16
    bf16 bits with in_type='bf16'.  axis 'row' -> one output per row; 'col' ->
    one output per column.  Returns (sum, sumsq) float32 arrays."""
    if in_type is None:
        in_type = "bf16" if X.dtype == np.uint16 else "fp32"
    X = np.ascontiguousarray(X, dtype=np.uint16 if in_type == "bf16" else np.float32)
    rows, cols = X.shape
    n_out = rows if axis == "row" else cols
    s = np.empty(n_out, dtype=np.float32)
    q = np.empty(n_out, dtype=np.float32)
    lib().or_reduce(1 if in_type == "bf16" else 0, 0 if axis == "row" else 1, rows, cols,
                    _ptr(X), cols, int(leaf_len), 1 if sq_fused else 0, _ptr(s), _ptr(q),
                    threads or default_threads())
    return s, q


# --------------------------------------------------------------------------
# descriptor JSON
# --------------------------------------------------------------------------
# The oracle reads the same descriptor text the library reads ("Taming
# Bitwise Behavior", section 4: the descriptor is a frozen record), with its
# own reader (Python's json module), and turns it into the specs the
# functions above take.  Fields it does not emulate must hold the value it
# does: a record asking for anything else is refused rather than computed in
# another order.
_GEMM_KEYS = {"version", "a_type", "b_type", "acc_type", "out_type", "partial_type", "merge_type", "mfma",
              "acc_update", "k_order", "short_turn", "k_slot_layout", "split_k", "cut_rule", "cut_unit", "cuts",
              "combine", "odd_rule", "rounding_point", "epilogue", "mfma_profile_hash", "schedule"}
_REDUCE_KEYS = {"version", "in_type", "acc_type", "out_type", "op", "axis", "leaf_len", "leaf_order", "sq_fma",
                "tree", "odd_rule", "schedule"}
# the one value the oracle emulates for each field it does not vary
_GEMM_FIXED = {"version": 1, "acc_update": "IN_MFMA", "k_order": "ASCENDING", "short_turn": "LAST",
               "k_slot_layout": "CONTIGUOUS", "partial_type": "fp32", "merge_type": "fp32",
               "odd_rule": "CARRY_LAST", "rounding_point": "AFTER_COMBINE_RNE"}
_REDUCE_FIXED = {"version": 1, "acc_type": "fp32", "out_type": "fp32", "leaf_order": "SEQUENTIAL_NO_SEED",
                 "tree": "BALANCED", "odd_rule": "CARRY_LAST"}


def _fnv1a64(data):
    h = 0xCBF29CE484222325
    for b in data:
        h = ((h ^ b) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def profile_models_hash(profile):
    """FNV-1a 64 of the canonical JSON of a probe profile's measured models
    (the hash a descriptor carries as mfma_profile_hash)."""
    import json as _json
    canon = _json.dumps(profile.get("models", {}), sort_keys=True, separators=(",", ":"))
    return _fnv1a64(canon.encode())


def desc_from_json(text, profile):
    """Descriptor JSON text -> (gemm spec or None, reduce spec or None) for
    gemm_bf16 / w8a8_pow2 / reduce.  `profile` is the probe's profile dict:
    its models give the instruction model, and its hash must equal the
    record's mfma_profile_hash (when the record names one)."""
    import json as _json
    doc = _json.loads(text)
    if not isinstance(doc, dict) or set(doc) - {"gemm", "reduce"}:
        raise ValueError("the document holds 'gemm' and/or 'reduce' only")
    g = r = None
    if "gemm" in doc:
        src = doc["gemm"]
        if set(src) - _GEMM_KEYS:
            raise ValueError(f"unknown gemm keys {sorted(set(src) - _GEMM_KEYS)}")
        for k, v in _GEMM_FIXED.items():
            if k in src and src[k] != v:
                raise ValueError(f"the oracle emulates {k} = {v!r} only, not {src[k]!r}")
        if src.get("combine", "BALANCED_NEIGHBOURS_FIRST") not in COMBINE:
            raise ValueError(f"unknown combine {src['combine']!r}")
        if "mfma_profile_hash" in src and int(src["mfma_profile_hash"], 16) != profile_models_hash(profile):
            raise ValueError("the record's mfma_profile_hash is not this profile's")
        mfma = src.get("mfma", "F32_32X32X16_BF16")
        g = {"mfma": mfma, "split_k": int(src.get("split_k", 1)),
             "cut_rule": src.get("cut_rule", "UNIT256_REMAINDER_LAST"), "cut_unit": int(src.get("cut_unit", 256)),
             "combine": src.get("combine", "BALANCED_NEIGHBOURS_FIRST"), "out_type": src.get("out_type", "bf16"),
             "epilogue": src.get("epilogue", "NONE")}
        if g["cut_rule"] not in ("UNIT256_REMAINDER_LAST", "EXPLICIT"):
            raise ValueError(f"unknown cut_rule {g['cut_rule']!r}")
        if "cuts" in src:
            g["cuts"] = [int(c) for c in src["cuts"]]
        if mfma in INSTR_K:   # the bf16 instructions: the measured model of one instruction
            g["mfma_model"] = profile["models"][mfma]
    if "reduce" in doc:
        src = doc["reduce"]
        if set(src) - _REDUCE_KEYS:
            raise ValueError(f"unknown reduce keys {sorted(set(src) - _REDUCE_KEYS)}")
        for k, v in _REDUCE_FIXED.items():
            if k in src and src[k] != v:
                raise ValueError(f"the oracle emulates {k} = {v!r} only, not {src[k]!r}")
        r = {"in_type": src.get("in_type", "fp32"), "op": src.get("op", "sum_and_sumsq"),
             "axis": src.get("axis", "row"), "leaf_len": int(src.get("leaf_len", 32)),
             "sq_fused": src.get("sq_fma", "fused") == "fused"}
        if src.get("sq_fma", "fused") not in ("fused", "unfused"):
            raise ValueError(f"unknown sq_fma {src['sq_fma']!r}")
    return g, r
