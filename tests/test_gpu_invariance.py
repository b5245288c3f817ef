"""Identical descriptors give identical bytes whatever stream runs the call
and however many CUs its kernels land on.  In "GPU Mechanism" (sections 4.2
and 4.4) the SM count a library targets picks the tile, the split-K and a
reduction's block split, and with them the summation order; here the
descriptor fixes the order and the CU count never enters a plan.  Checked
for ten repeats, a second stream, and streams restricted to 32, 64 and 128
CUs (hipExtStreamCreateWithCUMask), on the bf16 GEMM at one split and at
four, the W8A8 GEMM, the GEMM with a fused column sum, and both reduction
axes."""
import ctypes as C

import numpy as np
import pytest

import synth
from gpu_util import print_case, require_gpu, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _hip_runtime():
    """The HIP runtime this process already uses (the copy torch loaded, which
    libbitgemm's calls go to as well)."""
    for line in open("/proc/self/maps"):
        if "libamdhip64" in line:
            return C.CDLL(line.split()[-1])
    raise RuntimeError("the HIP runtime is not loaded")


class MaskedStream:
    """A HIP stream whose kernels run on the first n CUs of the device mask
    (normal priority)."""

    def __init__(self, n_cu, total_cu):
        self.hip = _hip_runtime()
        words = (total_cu + 31) // 32
        mask = (C.c_uint32 * words)()
        for i in range(n_cu):
            mask[i // 32] |= 1 << (i % 32)
        self.handle = C.c_void_p()
        rc = self.hip.hipExtStreamCreateWithCUMask(C.byref(self.handle), C.c_uint32(words), mask)
        assert rc == 0, f"hipExtStreamCreateWithCUMask returned {rc}"

    def sync(self):
        assert self.hip.hipStreamSynchronize(self.handle) == 0

    def close(self):
        self.hip.hipStreamDestroy(self.handle)


def _workloads():
    """name -> fn(stream) returning the output bytes of one call on that
    stream (None: torch's current stream).  Inputs are uploaded once."""
    import torch
    import fixed_order_fp_amd as bg
    out = {}

    X = to_dev_u16(synth.bf16_normal(1003, (300, 2560)))
    W = to_dev_u16(synth.bf16_normal(2003, (1000, 2560), 0.0, 0.02))
    for S, otype in ((1, "bf16"), (4, "fp32")):
        d = bg.gemm_desc({"split_k": S, "out_type": otype})
        nws = bg.gemm_workspace_bytes(d, 300, 1000, 2560)

        def gemm(stream, d=d, nws=nws, otype=otype):
            Cc = torch.empty((300, 1000), dtype=torch.int16 if otype == "bf16" else torch.float32, device="cuda")
            ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
            torch.cuda.synchronize()
            bg.gemm_bf16(d, X, W, Cc, ws, stream=stream)
            return [Cc]
        out[f"gemm_bf16 S={S} {otype}"] = gemm

    # a deep remainder split: the plan runs the two-tile-shape split kernel
    Xd = to_dev_u16(synth.bf16_normal(1004, (300, 9728)))
    Wd = to_dev_u16(synth.bf16_normal(2004, (1000, 9728), 0.0, 0.02))
    d16 = bg.gemm_desc({"split_k": 16, "out_type": "fp32"})
    assert bg.gemm_bf16_plan(d16, 300, 1000, 9728)["last_bm"] > 0
    n16 = bg.gemm_workspace_bytes(d16, 300, 1000, 9728)

    def gemm_deep(stream):
        Cc = torch.empty((300, 1000), dtype=torch.float32, device="cuda")
        ws = torch.empty(n16, dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        bg.gemm_bf16(d16, Xd, Wd, Cc, ws, stream=stream)
        return [Cc]
    out["gemm_bf16 S=16 two tile shapes"] = gemm_deep

    a_q, w_q, a_s, w_s = synth.w8a8_input(M=256, N=768, K=2048)
    dA, dW = torch.from_numpy(a_q).cuda(), torch.from_numpy(w_q).cuda()
    dsa, dsw = torch.from_numpy(a_s).cuda(), torch.from_numpy(w_s).cuda()
    d8 = bg.gemm_desc(dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32",
                           out_type="bf16", epilogue="W8A8_POW2", split_k=1))

    def w8a8(stream):
        Y = torch.empty((256, 768), dtype=torch.int16, device="cuda")
        acc = torch.empty((256, 768), dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        bg.gemm_w8a8_pow2(d8, dA, dW, dsa, dsw, Y, acc, stream=stream)
        return [Y, acc]
    out["w8a8"] = w8a8

    dg = bg.gemm_desc({"out_type": "bf16"})
    rd = bg.reduce_desc({"in_type": "fp32", "axis": "col"})
    nrw = bg.gemm_bf16_reduce_workspace_bytes(dg, rd, 300, 1000, 2560)

    def gemm_col_sum(stream):
        Cc = torch.empty((300, 1000), dtype=torch.int16, device="cuda")
        s = torch.empty(1000, dtype=torch.float32, device="cuda")
        q = torch.empty(1000, dtype=torch.float32, device="cuda")
        ws = torch.empty(nrw // 4 + 4, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        bg.gemm_bf16_reduce(dg, rd, X, W, Cc, s, q, ws, stream=stream)
        return [Cc, s, q]
    out["gemm_bf16_reduce col"] = gemm_col_sum

    R = torch.from_numpy(synth.f32_normal(1002, (512, 8192))).cuda()
    Ccol = to_dev_u16(synth.bf16_normal(2002, (8192, 1024), 0.0, 0.1))
    for axis, Xr, itype in (("row", R, "fp32"), ("col", Ccol, "bf16")):
        dr = bg.reduce_desc({"in_type": itype, "axis": axis})
        rows, cols = Xr.shape
        n_out = rows if axis == "row" else cols
        nws = bg.reduce_workspace_bytes(dr, rows, cols)

        def red(stream, dr=dr, Xr=Xr, n_out=n_out, nws=nws):
            s = torch.empty(n_out, dtype=torch.float32, device="cuda")
            q = torch.empty(n_out, dtype=torch.float32, device="cuda")
            ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
            torch.cuda.synchronize()
            bg.reduce_tree(dr, Xr, s, q, ws, stream=stream)
            return [s, q]
        out[f"reduce_tree {axis}"] = red
    return out


def _bytes(tensors):
    return [t.cpu().numpy().tobytes() for t in tensors]


def test_repeats_streams_and_cu_masks_do_not_move_bits():
    import torch
    total = torch.cuda.get_device_properties(0).multi_processor_count
    work = _workloads()
    ref = {}
    for name, fn in work.items():
        print_case("invariance reference", name)
        r = fn(None)
        torch.cuda.synchronize()
        ref[name] = _bytes(r)
        for rep in range(10):
            got = fn(None)
            torch.cuda.synchronize()
            assert _bytes(got) == ref[name], f"{name}: repeat {rep} differs"
    side = torch.cuda.Stream()
    for name, fn in work.items():
        print_case("invariance second stream", name)
        got = fn(side.cuda_stream)
        side.synchronize()
        assert _bytes(got) == ref[name], f"{name}: second stream differs"
    for n_cu in (32, 64, 128):
        ms = MaskedStream(n_cu, total)
        try:
            for name, fn in work.items():
                print_case("invariance CU mask", n_cu, name)
                got = fn(ms.handle.value)
                ms.sync()
                assert _bytes(got) == ref[name], f"{name}: {n_cu} CUs differ"
        finally:
            ms.close()


def test_cu_mask_takes_effect():
    """The masks above restrict the kernels for real: a GEMM with 256
    workgroups of one round (1024 x 2048 x 2560) runs several times longer on
    a 32-CU stream than on a stream masked to every CU."""
    import torch
    import fixed_order_fp_amd as bg
    total = torch.cuda.get_device_properties(0).multi_processor_count
    X = to_dev_u16(synth.bf16_normal(7, (1024, 2560)))
    W = to_dev_u16(synth.bf16_normal(8, (2048, 2560), 0.0, 0.02))
    Cc = torch.empty((1024, 2048), dtype=torch.int16, device="cuda")
    d = bg.gemm_desc({"out_type": "bf16"})
    torch.cuda.synchronize()
    times = {}
    for n_cu in (total, 32):
        ms = MaskedStream(n_cu, total)
        hip = ms.hip
        try:
            e0, e1 = C.c_void_p(), C.c_void_p()
            assert hip.hipEventCreate(C.byref(e0)) == 0 and hip.hipEventCreate(C.byref(e1)) == 0
            for _ in range(3):
                bg.gemm_bf16(d, X, W, Cc, None, stream=ms.handle.value)
            assert hip.hipEventRecord(e0, ms.handle) == 0
            for _ in range(10):
                bg.gemm_bf16(d, X, W, Cc, None, stream=ms.handle.value)
            assert hip.hipEventRecord(e1, ms.handle) == 0
            assert hip.hipEventSynchronize(e1) == 0
            t = C.c_float()
            assert hip.hipEventElapsedTime(C.byref(t), e0, e1) == 0
            times[n_cu] = t.value
            hip.hipEventDestroy(e0)
            hip.hipEventDestroy(e1)
        finally:
            ms.close()
    print_case("CU mask timing (ms per 10 calls)", times)
    assert times[32] > 3.0 * times[total], times
