"""Shared helpers for the test suite (no method arithmetic here)."""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svlm.h")


def declared_symbols():
    """Function names declared in include/svlm.h."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w\s\*]*?)\b(svlm_\w+)\s*\(", text, re.M)))


def dev_bf16(x: np.ndarray):
    """fp32 array holding bf16 values -> torch bf16 on cuda:0 (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")
    out = t.to(torch.bfloat16)
    assert torch.equal(out.float(), t), "input values are not bf16-representable"
    return out


def row_rel_err(o, ref):
    """max over rows of max_d |o - ref| / max_d |ref| (rows = all but the last axis)."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(o - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max())


def log(msg):
    print(msg, flush=True)
