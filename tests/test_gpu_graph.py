"""The order-fixed calls captured in a HIP graph: every replay must give the
eager call's bits.  Replays are separated by unrelated eager work and
synchronisations, and each one is checked (the library issues no memset, so
a replay has only kernel nodes)."""
import numpy as np
import pytest

import synth
from gpu_util import print_case, require_gpu, to_dev_u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _replays_match(fn, outs, torch, n=4):
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    for i in range(n):
        for o in outs:
            o.fill_(-1)
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int32) if o.dtype == torch.float32 else o,
                               e.view(torch.int32) if e.dtype == torch.float32 else e), f"replay {i}"


def test_gemm_split_k_graph():
    import torch
    import fixed_order_fp_amd as bg
    print_case("graph gemm S=4")
    A, B = synth.gemm_splitk_sweep()
    A, B = A[:64], B[:512]
    d = bg.gemm_desc({"split_k": 4, "out_type": "bf16"})
    dA, dB = to_dev_u16(A), to_dev_u16(B)
    C = torch.empty((64, 512), dtype=torch.int16, device="cuda")
    ws = torch.empty(bg.gemm_workspace_bytes(d, 64, 512, A.shape[1]), dtype=torch.uint8, device="cuda")
    fn = lambda: bg.gemm_bf16(d, dA, dB, C, ws)  # noqa: E731
    fn()
    _replays_match(fn, [C], torch)


def test_reduce_col_graph():
    import torch
    import fixed_order_fp_amd as bg
    print_case("graph reduce col")
    Y = synth.reduce_cols_input(rows=2048, cols=1024)
    d = bg.reduce_desc({"in_type": "bf16", "op": "sum_and_sumsq", "axis": "col"})
    dY = torch.from_numpy(np.ascontiguousarray(Y).view(np.int16)).cuda()
    s = torch.empty(1024, dtype=torch.float32, device="cuda")
    q = torch.empty(1024, dtype=torch.float32, device="cuda")
    nws = bg.reduce_workspace_bytes(d, 2048, 1024)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    fn = lambda: bg.reduce_tree(d, dY, s, q, ws)  # noqa: E731
    fn()
    _replays_match(fn, [s, q], torch)


def test_w8a8_graph():
    import torch
    import fixed_order_fp_amd as bg
    print_case("graph w8a8")
    a_q, w_q, a_s, w_s = synth.w8a8_input(M=128, N=256, K=512)
    d = bg.gemm_desc(dict(mfma="I32_32X32X32_I8", a_type="int8", b_type="int8", acc_type="int32",
                          out_type="bf16", epilogue="W8A8_POW2"))
    dA, dW = torch.from_numpy(a_q).cuda(), torch.from_numpy(w_q).cuda()
    sa, sw = torch.from_numpy(a_s).cuda(), torch.from_numpy(w_s).cuda()
    Y = torch.empty((128, 256), dtype=torch.int16, device="cuda")
    acc = torch.empty((128, 256), dtype=torch.int32, device="cuda")
    fn = lambda: bg.gemm_w8a8_pow2(d, dA, dW, sa, sw, Y, acc)  # noqa: E731
    fn()
    _replays_match(fn, [Y, acc], torch)
