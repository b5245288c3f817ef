#!/usr/bin/env python3
"""Benchmark of the order-fixed hot path on one MI355X.

The headline line times the order-fixed bf16 GEMM C = A B^T of the
batch-invariance sweep at its largest batch (M=4000, N=9728, K=2560, one
descriptor: 32x32x16 bf16 MFMA, split-K 1, bf16 output rounded once), with the
inputs resident in HBM.  A step is one call of that GEMM.  Before timing, a
sample of outputs is checked bit for bit against the oracle.

The same JSON line also carries:
  roofline      the GEMM kernel's achieved TFLOP/s (algorithmic 2*M*N*K per
                launch / average launch time from HIP events on the launch
                stream) against the dense bf16 MFMA peak;
  cpu_baseline  the oracle timed on a bounded sample of the same outputs on
                the host cores;
  extra         the other workloads (smaller batches, the split-K sweep, the
                small split-K GEMM), each parity-sampled and timed the same
                way, and the free-order twin where it is built.

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("order-fixed bf16 GEMM TFLOP/s (bit-exact vs oracle), % MFMA peak, "
          "cost vs free order")
PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Gemm:
    """One order-fixed GEMM workload resident on the GPU."""

    def __init__(self, name, A, B, spec, torch, bg):
        self.name, self.torch, self.bg = name, torch, bg
        self.A_host, self.B_host = A, B
        self.spec = dict(spec)
        self.M, self.K = A.shape
        self.N = B.shape[0]
        self.desc = bg.gemm_desc(self.spec)
        import numpy as np
        self.dA = torch.from_numpy(A.view(np.int16)).cuda()
        self.dB = torch.from_numpy(B.view(np.int16)).cuda()
        out_bf16 = self.spec.get("out_type", "bf16") == "bf16"
        self.dC = torch.empty((self.M, self.N), dtype=torch.int16 if out_bf16 else torch.float32,
                              device="cuda")
        nws = bg.gemm_workspace_bytes(self.desc, self.M, self.N, self.K)
        self.ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None

    def run(self):
        self.bg.gemm_bf16(self.desc, self.dA, self.dB, self.dC, self.ws)

    def flops(self):
        return 2.0 * self.M * self.N * self.K

    def bytes(self):
        out = 2 if self.spec.get("out_type", "bf16") == "bf16" else 4
        S = int(self.spec.get("split_k", 1))
        ws = 2 * (S - 1) * self.M * self.N * 4 if S > 1 else 0
        return 2.0 * (self.M + self.N) * self.K + out * self.M * self.N + ws

    def parity(self, n_points=256, seed=0):
        """Bit-compare sampled outputs with the oracle."""
        import numpy as np
        import oracle
        self.run()
        self.torch.cuda.synchronize()
        C = self.dC.cpu().numpy()
        rng = np.random.default_rng(seed)
        mi = rng.integers(0, self.M, n_points)
        ni = rng.integers(0, self.N, n_points)
        model = self.bg.load_profile()["models"][self.spec.get("mfma", "F32_32X32X16_BF16")]
        ref = oracle.gemm_bf16_points(dict(self.spec, mfma_model=model), self.A_host, self.B_host, mi, ni)
        got = C[mi, ni]
        bad = int(np.sum(got.view(ref.dtype) != ref)) if ref.dtype == np.uint16 else \
            int(np.sum(got.view(np.uint32) != ref.view(np.uint32)))
        return {"sampled": int(n_points), "mismatches": bad}


def time_steps(fn, steps, warmup, torch):
    """Warm up, then time exactly `steps` calls between synchronisations with
    HIP events recorded on the stream the kernels are launched on."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def cpu_baseline(g, budget_s=12.0):
    """The oracle, as it stands, on a bounded sample of the headline GEMM's
    outputs, on every host core it is given."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    model = g.bg.load_profile()["models"][g.spec.get("mfma", "F32_32X32X16_BF16")]
    desc = dict(g.spec, mfma_model=model)
    rng = np.random.default_rng(1)
    done, t_total, chunk = 0, 0.0, 2000
    while t_total < budget_s:
        mi = rng.integers(0, g.M, chunk)
        ni = rng.integers(0, g.N, chunk)
        t0 = time.perf_counter()
        oracle.gemm_bf16_points(desc, g.A_host, g.B_host, mi, ni, threads=threads)
        dt = time.perf_counter() - t0
        t_total += dt
        done += chunk
        if dt < budget_s / 8:
            chunk *= 2
    tflops = 2.0 * g.K * done / t_total / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{done} outputs of the M=4000 N=9728 K=2560 GEMM, {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported here "
              "(the method shards by output columns or rows with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import fixed_order_fp_amd as bg
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    log("bench: generating the batch-sweep workload")
    X, W = synth.gemm_batch_sweep(M=4000)
    head = Gemm("gemm_bf16 M=4000", X, W, {"mfma": "F32_32X32X16_BF16", "out_type": "bf16"}, torch, bg)
    par = head.parity(512)
    log(f"bench: parity {par}")
    ms, wall = time_steps(head.run, args.steps, args.warmup, torch)
    tflops = head.flops() / (ms * 1e-3) / 1e12
    log(f"bench: {ms:.4f} ms per call, {tflops:.1f} TFLOP/s")

    line = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "order-fixed bf16 GEMM C=A*B^T, batch-invariance sweep at M=4000 "
                               "(N=9728, K=2560), 32x32x16 bf16 MFMA, split-K 1, bf16 out",
                   "M": 4000, "N": 9728, "K": 2560, "split_k": 1, "mfma": "F32_32X32X16_BF16",
                   "out": "bf16"},
        "parity": par,
        "roofline": {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None},
    }
    del wall

    extra = {}
    if not args.no_extra:
        for M in (1, 8, 64, 512):
            g = Gemm(f"gemm_bf16 M={M}", X[:M].copy(), W, {"mfma": "F32_32X32X16_BF16", "out_type": "bf16"},
                     torch, bg)
            p = g.parity(128)
            t, _ = time_steps(g.run, args.steps, args.warmup, torch)
            extra[f"batch_sweep_M{M}"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(g.flops() / t / 1e9, 2),
                                          "GB/s": round(g.bytes() / t / 1e6, 1), "parity": p}
            log(f"bench: M={M}: {t * 1e3:.2f} us")
        A4, W4 = synth.gemm_splitk_sweep()
        for S in (1, 2, 4, 8, 16):
            g = Gemm(f"splitk S={S}", A4, W4, {"mfma": "F32_32X32X16_BF16", "split_k": S, "out_type": "fp32"},
                     torch, bg)
            p = g.parity(128)
            t, _ = time_steps(g.run, args.steps, args.warmup, torch)
            extra[f"splitk_S{S}"] = {"us": round(t * 1e3, 2), "TFLOP/s": round(g.flops() / t / 1e9, 2),
                                     "GB/s": round(g.bytes() / t / 1e6, 1), "parity": p}
            log(f"bench: split-K S={S}: {t * 1e3:.2f} us")
        A1, B1 = synth.gemm_small()
        g = Gemm("small", A1, B1, {"mfma": "F32_32X32X16_BF16", "split_k": 2, "cut_rule": "EXPLICIT",
                                   "cuts": [0, 256, 512], "out_type": "fp32"}, torch, bg)
        p = g.parity(256)
        t, _ = time_steps(g.run, args.steps, args.warmup, torch)
        extra["small_32x64x512_S2"] = {"us": round(t * 1e3, 2), "parity": p}
    if extra:
        line["extra"] = extra

    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(head)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
