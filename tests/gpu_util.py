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


# E4M3 runs: the absolute bar follows from the cosine bar. cos >= 0.999 bounds the
# difference RMS by sqrt(2 * 0.001) ~ 4.5% of the row RMS; over D ~ 1000 roughly
# independent components the largest sits near 4 sigma, so 0.2 x the row RMS.
E4M3_ABS_OF_RMS = 0.2


def check_pooled(got, want, label, e4m3=False):
    got = np.asarray(got, np.float64)
    cos = row_cos(got, want)
    err = np.abs(got - want).max(1) if len(want) else np.zeros(0)
    bar = (E4M3_ABS_OF_RMS * np.sqrt((want ** 2).mean(1)) if e4m3 else np.full(len(want), ABS_MAX))
    say(f"[{label}] rows {len(want)}: min cos {cos.min() if len(cos) else 1:.6f}, "
        f"max |diff| {err.max() if len(err) else 0:.3e} (bar {bar.min() if len(bar) else 0:.3e})")
    assert cos.min() >= COS_MIN, (label, cos.min())
    assert np.all(err <= bar), (label, err.max())
    return cos, err
