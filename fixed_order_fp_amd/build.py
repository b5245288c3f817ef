"""Build libbitgemm.so for gfx950 in-tree with hipcc.

Every HIP source is compiled with -ffp-contract=off (no multiply-add is fused
unless the code says fma) and with packed fp32 instructions disabled; the
MFMA profile hash the descriptors must carry is baked in from
profiles/gfx950.json.
"""
import concurrent.futures as cf
import hashlib  # noqa: F401  (kept for callers that want a content digest)
import json
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbitgemm.so")
PROFILE = os.path.join(HERE, "profiles", "gfx950.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["bg_api.hip", "bg_desc_json.cpp", "bg_probe.hip", "bg_gemm_bf16.hip", "bg_reduce.hip", "bg_w8a8.hip",
           "bg_quant.hip", "bg_ozaki.hip"]

FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def fnv1a64(data: bytes) -> int:
    h = 0xCBF29CE484222325
    for b in data:
        h = ((h ^ b) * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h


def profile_hash(path=PROFILE) -> int:
    """FNV-1a 64 of the canonical JSON of the profile's measured models."""
    with open(path) as f:
        prof = json.load(f)
    canon = json.dumps(prof.get("models", {}), sort_keys=True, separators=(",", ":"))
    return fnv1a64(canon.encode())


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in (r.stderr or "").splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    return obj, warn


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    extra = [f"-DBG_PROFILE_HASH=0x{profile_hash():016x}ull"]
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1, 16)
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, extra), SOURCES))
    objs = []
    for obj, warn in results:
        objs.append(obj)
        if warn and verbose:
            print(warn, file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
