"""bg_gemm_bf16_noalloc (split-K partials in the library's static scratch)
against bg_gemm_bf16 with a caller workspace, through the C ABI: the same
descriptor must give the same bytes, on two calls in a row (the second
smaller, so that the scratch still holds the first call's partials), and a
call needing more than the scratch is refused before anything runs."""
import numpy as np
import pytest

import synth
from gpu_util import print_case, require_gpu, to_dev_u16

pytestmark = pytest.mark.gpu


def _pair(bg, torch, spec, A, B, out):
    d = bg.gemm_desc(spec, out_type=out)
    M, K = A.shape
    N = B.shape[0]
    dA, dB = to_dev_u16(A), to_dev_u16(B)
    dt = torch.float32 if out == "fp32" else torch.int16
    ref = torch.full((M, N), -1, dtype=dt, device="cuda")
    got = torch.full((M, N), -2, dtype=dt, device="cuda")
    nws = bg.gemm_workspace_bytes(d, M, N, K)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    bg.gemm_bf16(d, dA, dB, ref, ws)
    bg.gemm_bf16_noalloc(d, dA, dB, got)
    torch.cuda.synchronize()
    view = np.uint32 if out == "fp32" else np.uint16
    return got.cpu().numpy().view(view), ref.cpu().numpy().view(view), nws


def test_noalloc_matches_the_workspace_entry_point():
    require_gpu()
    import torch
    import fixed_order_fp_amd as bg
    # call 1: the split-K sweep workload at S = 16 (42 MB of partials)
    A, B = synth.gemm_splitk_sweep()
    print_case("noalloc 256x2560x9728 S=16 fp32")
    got, ref, nws = _pair(bg, torch, {"split_k": 16}, A, B, "fp32")
    assert nws == 16 * 256 * 2560 * 4
    assert np.array_equal(got, ref)
    # call 2, smaller: ragged 70 x 136 x 2048, S = 4, bf16 out
    A2 = synth.bf16_spread(81, (70, 2048), -20, 20)
    B2 = synth.bf16_spread(82, (136, 2048), -20, 20)
    print_case("noalloc 70x136x2048 S=4 bf16")
    got, ref, _ = _pair(bg, torch, {"split_k": 4}, A2, B2, "bf16")
    assert np.array_equal(got, ref)
    # S = 1 takes no scratch
    print_case("noalloc 70x136x2048 S=1 bf16")
    got, ref, nws = _pair(bg, torch, {}, A2, B2, "bf16")
    assert nws == 0 and np.array_equal(got, ref)


def test_noalloc_refuses_more_than_the_scratch():
    require_gpu()
    import torch
    import fixed_order_fp_amd as bg
    print_case("noalloc refusal 4096x4096 S=2")
    d = bg.gemm_desc({"split_k": 2}, out_type="fp32")
    A = torch.zeros((4096, 512), dtype=torch.int16, device="cuda")
    B = torch.zeros((4096, 512), dtype=torch.int16, device="cuda")
    C = torch.full((4096, 4096), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(bg.BgError, match="BG_E_WORKSPACE"):
        bg.gemm_bf16_noalloc(d, A, B, C)   # 134 MB of partials > 64 MiB
    torch.cuda.synchronize()
    assert bool((C == 7.0).all())          # nothing ran
