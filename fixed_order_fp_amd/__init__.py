"""Python binding of libbitgemm (argument marshalling only).

Every call goes straight to the C ABI in include/bitgemm.h; every step of the
hot path runs in the library's HIP kernels.  PyTorch provides device memory
and the current stream.  If libbitgemm.so has not been built, the first call
raises: there is no fallback of any kind.
"""
import ctypes as C
import json
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbitgemm.so")
PROFILE_PATH = os.path.join(HERE, "profiles", "gfx950.json")

BG_MAX_SPLIT = 64

# enums (values as in bitgemm.h)
FP32, BF16, INT8, INT32 = 0, 1, 2, 3
MFMA = {"F32_32X32X16_BF16": 0, "F32_16X16X32_BF16": 1, "I32_32X32X32_I8": 2, "I32_16X16X64_I8": 3}
INSTR_K = {"F32_32X32X16_BF16": 16, "F32_16X16X32_BF16": 32, "I32_32X32X32_I8": 32, "I32_16X16X64_I8": 64}
CUT_RULE = {"UNIT256_REMAINDER_LAST": 0, "EXPLICIT": 1}
COMBINE = {"BALANCED_NEIGHBOURS_FIRST": 0, "SEQUENTIAL": 1}
DTYPE = {"fp32": FP32, "bf16": BF16, "int8": INT8, "int32": INT32}
EPILOGUE = {"NONE": 0, "W8A8_POW2": 1}
RED_OP = {"sum": 1, "sumsq": 2, "sum_and_sumsq": 3}
AXIS = {"row": 0, "col": 1}
SQ_FMA = {"fused": 0, "unfused": 1}

STATUS = {0: "BG_OK", 1: "BG_E_INVALID", 2: "BG_E_UNSUPPORTED", 3: "BG_E_WORKSPACE",
          4: "BG_E_ALIGN", 5: "BG_E_ARCH", 6: "BG_E_PROFILE", 7: "BG_E_HIP"}


class GemmSchedule(C.Structure):
    _fields_ = [("bm", C.c_int32), ("bn", C.c_int32), ("bk", C.c_int32),
                ("waves_m", C.c_int32), ("waves_n", C.c_int32), ("load_path", C.c_int32),
                ("group_m", C.c_int32), ("stages", C.c_int32), ("last_bm", C.c_int32),
                ("last_bn", C.c_int32), ("last_waves_m", C.c_int32), ("last_waves_n", C.c_int32),
                ("last_stages", C.c_int32)]


class GemmDesc(C.Structure):
    _fields_ = [("version", C.c_uint32), ("a_type", C.c_uint32), ("b_type", C.c_uint32),
                ("acc_type", C.c_uint32), ("out_type", C.c_uint32), ("mfma", C.c_uint32),
                ("acc_update", C.c_uint32), ("k_order", C.c_uint32), ("short_turn", C.c_uint32),
                ("k_slot_layout", C.c_uint32), ("split_k", C.c_uint32), ("cut_rule", C.c_uint32),
                ("cut_unit", C.c_uint32), ("cuts", C.c_int64 * (BG_MAX_SPLIT + 1)),
                ("partial_type", C.c_uint32), ("merge_type", C.c_uint32), ("combine", C.c_uint32),
                ("odd_rule", C.c_uint32), ("rounding_point", C.c_uint32), ("epilogue", C.c_uint32),
                ("mfma_profile_hash", C.c_uint64), ("sched", GemmSchedule)]


class ReduceSchedule(C.Structure):
    _fields_ = [("leaves_per_wg", C.c_int32), ("cols_per_wg", C.c_int32),
                ("reserved0", C.c_int32), ("reserved1", C.c_int32)]


class ReduceDesc(C.Structure):
    _fields_ = [("version", C.c_uint32), ("in_type", C.c_uint32), ("acc_type", C.c_uint32),
                ("op", C.c_uint32), ("axis", C.c_uint32), ("leaf_len", C.c_uint32),
                ("leaf_order", C.c_uint32), ("sq_fma", C.c_uint32), ("tree", C.c_uint32),
                ("odd_rule", C.c_uint32), ("out_type", C.c_uint32), ("sched", ReduceSchedule)]


class BgError(RuntimeError):
    def __init__(self, status, message):
        self.status = STATUS.get(status, status)
        super().__init__(f"{self.status}: {message}")


_lib = None

_SYMBOLS = {
    # name: (restype, argtypes)
    "bg_abi_version": (C.c_int, []),
    "bg_status_str": (C.c_char_p, [C.c_int]),
    "bg_last_error": (C.c_char_p, []),
    "bg_profile_hash": (C.c_uint64, []),
    "bg_desc_default_gemm": (C.c_int, [C.c_void_p]),
    "bg_desc_default_reduce": (C.c_int, [C.c_void_p]),
    "bg_desc_signature": (C.c_int, [C.c_void_p, C.c_void_p]),
    "bg_reduce_desc_signature": (C.c_int, [C.c_void_p, C.c_void_p]),
    "bg_desc_from_json": (C.c_int, [C.c_char_p, C.c_void_p, C.c_void_p]),
    "bg_desc_to_json": (C.c_int, [C.c_void_p, C.c_void_p, C.c_char_p, C.c_size_t, C.c_void_p]),
    "bg_gemm_split_cuts": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p]),
    "bg_gemm_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p]),
    "bg_gemm_bf16": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                               C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_size_t,
                               C.c_void_p]),
    "bg_gemm_bf16_plan": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p]),
    "bg_gemm_bf16_noalloc": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                                       C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p]),
    "bg_gemm_w8a8_pow2": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                                    C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64,
                                    C.c_void_p, C.c_int64, C.c_void_p]),
    "bg_gemm_bf16_reduce_workspace_bytes": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64,
                                                      C.c_void_p]),
    "bg_gemm_bf16_reduce": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int64, C.c_int64, C.c_int64, C.c_void_p,
                                      C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "bg_gemm_ozaki_workspace_bytes": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_void_p]),
    "bg_gemm_ozaki": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_uint32, C.c_void_p, C.c_int64, C.c_void_p,
                                C.c_int64, C.c_uint32, C.c_void_p, C.c_int64, C.c_void_p, C.c_size_t,
                                C.c_void_p]),
    "bg_quantize_act_int8": (C.c_int, [C.c_int64, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_int64,
                                       C.c_void_p, C.c_void_p]),
    "bg_requantize_weights_pow2": (C.c_int, [C.c_int64, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p,
                                             C.c_uint32, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p]),
    "bg_reduce_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p]),
    "bg_reduce_tree": (C.c_int, [C.c_void_p, C.c_int64, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p,
                                 C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "bg_bench_gemm_bf16_free": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                                          C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_int32,
                                          C.c_void_p]),
    "bg_bench_gemm_bf16_two_chains": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int64,
                                                C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p]),
    "bg_bench_gemm_w8a8_free": (C.c_int, [C.c_int64, C.c_int64, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p,
                                          C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int64, C.c_void_p]),
    "bg_bench_reduce_free": (C.c_int, [C.c_uint32, C.c_uint32, C.c_int64, C.c_int64, C.c_void_p,
                                       C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p]),
    "bg_probe_mfma": (C.c_int, [C.c_uint32, C.c_int64, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                C.c_void_p]),
}


def lib():
    """Load libbitgemm.so (built in-tree by build.py).  Raises if missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run fixed_order_fp_amd/build.py "
                               "(there is no fallback path)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SYMBOLS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SYMBOLS)


def _check(status):
    if status != 0:
        msg = lib().bg_last_error().decode(errors="replace")
        raise BgError(status, msg)


def _ptr(t):
    """Device (or host) address of a torch tensor / numpy array, or None."""
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return C.c_void_p(t.data_ptr())
    return C.c_void_p(t.ctypes.data)


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


# ----------------------------------------------------------------------------
# profile and descriptors
# ----------------------------------------------------------------------------


def load_profile(path=PROFILE_PATH):
    with open(path) as f:
        return json.load(f)


def profile_hash():
    return int(lib().bg_profile_hash())


def gemm_desc(spec=None, **overrides):
    """Build a GemmDesc from a descriptor dict (the JSON format the tests and
    the oracle share): mfma, split_k, cut_rule, cuts, cut_unit, combine,
    out_type, epilogue, a_type/b_type/acc_type, and an optional 'schedule'
    dict (bm, bn, bk, waves_m, waves_n, load_path, group_m, stages and the
    last split's last_bm, last_bn, last_waves_m, last_waves_n, last_stages).
    Unset fields keep the library
    defaults; the profile hash is the library's."""
    spec = dict(spec or {}, **overrides)
    d = GemmDesc()
    _check(lib().bg_desc_default_gemm(C.byref(d)))
    if "mfma" in spec:
        d.mfma = MFMA[spec["mfma"]]
    if "split_k" in spec:
        d.split_k = int(spec["split_k"])
    if "cut_rule" in spec:
        d.cut_rule = CUT_RULE[spec["cut_rule"]]
    if spec.get("cuts") is not None:
        for i, c in enumerate(spec["cuts"]):
            d.cuts[i] = int(c)
    if "cut_unit" in spec:
        d.cut_unit = int(spec["cut_unit"])
    if "combine" in spec:
        d.combine = COMBINE[spec["combine"]]
    if "out_type" in spec:
        d.out_type = DTYPE[spec["out_type"]]
    for f in ("a_type", "b_type", "acc_type", "partial_type", "merge_type"):
        if f in spec:
            setattr(d, f, DTYPE[spec[f]])
    if "epilogue" in spec:
        d.epilogue = EPILOGUE[spec["epilogue"]]
    for f in ("acc_update", "short_turn", "k_slot_layout", "version"):
        if f in spec:
            setattr(d, f, int(spec[f]))
    if "mfma_profile_hash" in spec:
        d.mfma_profile_hash = int(spec["mfma_profile_hash"])
    for k, v in (spec.get("schedule") or {}).items():
        setattr(d.sched, k, int(v))
    return d


def reduce_desc(spec=None, **overrides):
    spec = dict(spec or {}, **overrides)
    d = ReduceDesc()
    _check(lib().bg_desc_default_reduce(C.byref(d)))
    if "in_type" in spec:
        d.in_type = DTYPE[spec["in_type"]]
    if "op" in spec:
        d.op = RED_OP[spec["op"]]
    if "axis" in spec:
        d.axis = AXIS[spec["axis"]]
    if "leaf_len" in spec:
        d.leaf_len = int(spec["leaf_len"])
    if "sq_fma" in spec:
        d.sq_fma = SQ_FMA[spec["sq_fma"]]
    for k, v in (spec.get("schedule") or {}).items():
        setattr(d.sched, k, int(v))
    return d


def desc_from_json(text):
    """(GemmDesc, ReduceDesc) from descriptor JSON text, read by the library."""
    g, r = GemmDesc(), ReduceDesc()
    _check(lib().bg_desc_from_json(text.encode() if isinstance(text, str) else text, C.byref(g), C.byref(r)))
    return g, r


def desc_to_json(gemm=None, reduce=None):
    """Descriptor JSON text of a GemmDesc and/or ReduceDesc, written by the library."""
    n = C.c_size_t(0)
    gp = C.byref(gemm) if gemm is not None else None
    rp = C.byref(reduce) if reduce is not None else None
    lib().bg_desc_to_json(gp, rp, None, 0, C.byref(n))   # asks for the length
    buf = C.create_string_buffer(n.value + 1)
    _check(lib().bg_desc_to_json(gp, rp, buf, n.value + 1, C.byref(n)))
    return buf.value.decode()


def signature(desc):
    sig = (C.c_uint64 * 2)()
    if isinstance(desc, ReduceDesc):
        _check(lib().bg_reduce_desc_signature(C.byref(desc), sig))
    else:
        _check(lib().bg_desc_signature(C.byref(desc), sig))
    return (int(sig[0]), int(sig[1]))


def split_cuts(desc, K):
    cuts = (C.c_int64 * (BG_MAX_SPLIT + 1))()
    _check(lib().bg_gemm_split_cuts(C.byref(desc), int(K), cuts))
    return [int(cuts[i]) for i in range(desc.split_k + 1)]


def gemm_workspace_bytes(desc, M, N, K):
    n = C.c_size_t()
    _check(lib().bg_gemm_workspace_bytes(C.byref(desc), int(M), int(N), int(K), C.byref(n)))
    return int(n.value)


def reduce_workspace_bytes(desc, rows, cols):
    n = C.c_size_t()
    _check(lib().bg_reduce_workspace_bytes(C.byref(desc), int(rows), int(cols), C.byref(n)))
    return int(n.value)


# ----------------------------------------------------------------------------
# entry points (torch tensors on the GPU)
# ----------------------------------------------------------------------------


def gemm_bf16(desc, A, B, C_out, ws=None, stream=None):
    """C_out = A B^T under desc.  A [M][K], B [N][K] bf16 (torch.bfloat16 or
    int16 bit patterns); C_out fp32 or bf16 [M][N]; ws a uint8 tensor of at
    least gemm_workspace_bytes() bytes (or None when 0)."""
    M, K = A.shape
    N = B.shape[0]
    _check(lib().bg_gemm_bf16(C.byref(desc), M, N, K, _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                              _ptr(C_out), C_out.stride(0), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def gemm_bf16_plan(desc, M, N, K):
    """The tiles bg_gemm_bf16 would launch for desc at M x N x K, as a
    schedule dict (host only)."""
    s = GemmSchedule()
    _check(lib().bg_gemm_bf16_plan(C.byref(desc), M, N, K, C.byref(s)))
    return {f: int(getattr(s, f)) for f, _ in GemmSchedule._fields_}


def gemm_bf16_noalloc(desc, A, B, C_out, stream=None):
    """C_out = A B^T under desc with the library's static scratch for split-K
    partials (no workspace argument)."""
    M, K = A.shape
    N = B.shape[0]
    _check(lib().bg_gemm_bf16_noalloc(C.byref(desc), M, N, K, _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                      _ptr(C_out), C_out.stride(0), _stream(stream)))


def gemm_w8a8_pow2(desc, A, W, a_scale, w_scale, Y, acc_out=None, stream=None):
    M, K = A.shape
    N = W.shape[0]
    _check(lib().bg_gemm_w8a8_pow2(C.byref(desc), M, N, K, _ptr(A), A.stride(0), _ptr(W), W.stride(0),
                                   _ptr(a_scale), _ptr(w_scale), _ptr(Y), Y.stride(0), _ptr(acc_out),
                                   0 if acc_out is None else acc_out.stride(0), _stream(stream)))


def gemm_bf16_reduce_workspace_bytes(desc, rdesc, M, N, K):
    n = C.c_size_t(0)
    _check(lib().bg_gemm_bf16_reduce_workspace_bytes(C.byref(desc), C.byref(rdesc), M, N, K, C.byref(n)))
    return n.value


def gemm_bf16_reduce(desc, rdesc, A, B, C_out, out_sum=None, out_sumsq=None, ws=None, stream=None):
    """C = A B^T (bf16) plus the fixed-order reduction rdesc of the fp32 C."""
    M, K = A.shape
    N = B.shape[0]
    _check(lib().bg_gemm_bf16_reduce(C.byref(desc), C.byref(rdesc), M, N, K, _ptr(A), A.stride(0), _ptr(B),
                                     B.stride(0), _ptr(C_out), C_out.stride(0), _ptr(out_sum), _ptr(out_sumsq),
                                     _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream)))


def gemm_ozaki_workspace_bytes(M, N, K):
    n = C.c_size_t(0)
    _check(lib().bg_gemm_ozaki_workspace_bytes(M, N, K, C.byref(n)))
    return n.value


def gemm_ozaki(A, B, C_out, in_type, out_type, ws, stream=None):
    """C = A B^T by the Ozaki scheme (int8 slices, exact integer products)."""
    M, K = A.shape
    N = B.shape[0]
    _check(lib().bg_gemm_ozaki(M, N, K, DTYPE[in_type], _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                               DTYPE[out_type], _ptr(C_out), C_out.stride(0), _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def quantize_act_int8(X, Q, a_scale, stream=None):
    """Per-token int8 quantisation: X fp32 [M][K] -> Q int8 [M][K], a_scale fp32 [M]."""
    M, K = X.shape
    _check(lib().bg_quantize_act_int8(M, K, _ptr(X), X.stride(0), _ptr(Q), Q.stride(0), _ptr(a_scale),
                                      _stream(stream)))


POW2 = {"nearest": 0, "ceil": 1}


def requantize_weights_pow2(W, w_scale, W2, w_scale2, mode="nearest", stream=None):
    """int8 W [N][K] with scales w_scale [N] -> W2, w_scale2 with power-of-two scales."""
    N, K = W.shape
    _check(lib().bg_requantize_weights_pow2(N, K, _ptr(W), W.stride(0), _ptr(w_scale), POW2[mode], _ptr(W2),
                                            W2.stride(0), _ptr(w_scale2), _stream(stream)))


def reduce_tree(desc, X, out_sum=None, out_sumsq=None, ws=None, stream=None):
    rows, cols = X.shape
    _check(lib().bg_reduce_tree(C.byref(desc), rows, cols, _ptr(X), X.stride(0), _ptr(out_sum),
                                _ptr(out_sumsq), _ptr(ws),
                                0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def bench_gemm_bf16_free(A, B, C_out, split_k=0, stream=None):
    M, K = A.shape
    N = B.shape[0]
    _check(lib().bg_bench_gemm_bf16_free(M, N, K, _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                         _ptr(C_out), C_out.stride(0), int(split_k), _stream(stream)))


def bench_gemm_bf16_two_chains(A, B, C_out, stream=None):
    """Free-order twin (bench only): C_out fp32 = A B^T with two interleaved
    accumulator chains per output, on the 128x128 tile with 64-deep k tiles."""
    M, K = A.shape
    N = B.shape[0]
    _check(lib().bg_bench_gemm_bf16_two_chains(M, N, K, _ptr(A), A.stride(0), _ptr(B), B.stride(0),
                                               _ptr(C_out), C_out.stride(0), _stream(stream)))


def bench_gemm_w8a8_free(A, W, a_scale, w_scale, Y, stream=None):
    M, K = A.shape
    N = W.shape[0]
    _check(lib().bg_bench_gemm_w8a8_free(M, N, K, _ptr(A), A.stride(0), _ptr(W), W.stride(0), _ptr(a_scale),
                                         _ptr(w_scale), _ptr(Y), Y.stride(0), _stream(stream)))


def bench_reduce_free(axis, in_type, X, out_sum=None, out_sumsq=None, stream=None):
    rows, cols = X.shape
    _check(lib().bg_bench_reduce_free(AXIS[axis], DTYPE[in_type], rows, cols, _ptr(X), X.stride(0),
                                      _ptr(out_sum), _ptr(out_sumsq), _stream(stream)))


def probe_mfma(mfma, n_cases, A, B, C_in, D, stream=None):
    """One instruction per case on crafted tiles (see bitgemm.h)."""
    _check(lib().bg_probe_mfma(MFMA[mfma] if isinstance(mfma, str) else int(mfma), int(n_cases),
                               _ptr(A), _ptr(B), _ptr(C_in), _ptr(D), _stream(stream)))
