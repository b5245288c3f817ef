"""Helpers shared by the GPU tests: device checks, host<->device copies of
bit patterns, and the descriptor dicts both sides read."""
import json
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILE = os.path.join(ROOT, "fixed_order_fp_amd", "profiles", "gfx950.json")


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    name = torch.cuda.get_device_properties(0).gcnArchName
    if not name.startswith("gfx950"):
        pytest.skip(f"needs gfx950, found {name}")


def to_dev_u16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16)).cuda()


def to_dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def from_dev_u16(t):
    return t.cpu().numpy().view(np.uint16)


def profile():
    with open(PROFILE) as f:
        return json.load(f)


def measured_model(instr):
    """The MFMA model the probe measured for `instr`, or skip when the profile
    has not been measured."""
    prof = profile()
    m = prof.get("models", {}).get(instr)
    if prof.get("status") != "measured" or m is None:
        pytest.skip("MFMA profile not measured yet")
    return m


def oracle_desc(spec, instr=None):
    """The oracle's view of a descriptor dict: the same fields plus the
    measured instruction model."""
    instr = instr or spec.get("mfma", "F32_32X32X16_BF16")
    d = dict(spec)
    d["mfma"] = instr
    d["mfma_model"] = measured_model(instr)
    return d


def print_case(*parts):
    print("CASE", *parts, flush=True)
