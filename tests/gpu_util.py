"""Helpers shared by the GPU tests (marshalling and comparison only)."""
import sys

import numpy as np

COS_MIN = 0.999   # pooled-embedding cosine bar, per row
ABS_MAX = 2e-2    # max |difference| bar over all elements (bf16 path)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_bytes(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def bf16_tensor(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def row_cos(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    num = (got * want).sum(1)
    den = np.linalg.norm(got, axis=1) * np.linalg.norm(want, axis=1)
    out = np.ones(len(got))
    nz = den > 0
    out[nz] = num[nz] / den[nz]
    both_zero = (np.linalg.norm(got, axis=1) == 0) & (np.linalg.norm(want, axis=1) == 0)
    out[~nz & ~both_zero] = 0.0
    return out


def check_pooled(got, want, label):
    cos = row_cos(got, want)
    err = float(np.abs(np.asarray(got, np.float64) - want).max()) if len(want) else 0.0
    say(f"[{label}] rows {len(want)}: min cos {cos.min() if len(cos) else 1:.6f}, max |diff| {err:.3e}")
    assert cos.min() >= COS_MIN, (label, cos.min())
    assert err <= ABS_MAX, (label, err)
    return cos, err
