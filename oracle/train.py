"""CPU oracle of one training step of the text encoder: the backward pass and the Adafactor update.

TEST INFRASTRUCTURE ONLY: imported by the tests, ``__graft_entry__.smoke`` and the CPU-baseline leg of
``bench.py``; the product package never imports it, and it shares no code with the HIP path.

* ``text_forward``: the encoder's forward pass written with float64 torch operations on the CPU, step
  for step as oracle.c writes it (byte gather; pre-norm blocks of RMSNorm, fused QKV projection, 1-axis
  rotary on q and k, bidirectional attention inside each item, output projection and residual, RMSNorm,
  SwiGLU and residual; final RMSNorm; the dense attention pool) -- "UForm" page, "Architecture & Goals",
  FAQ "Why attention pooling instead of mean pooling?". Its output is pinned to oracle.c's.
* ``text_backward``: gradients of <pooled, d_pooled> with respect to every parameter by torch autograd
  over that float64 forward (a library primitive standing for the chain rule; pinned by finite
  differences).
* ``adafactor``: one Adafactor update ("UForm" page, "Adafactor Optimizer" and "Precision by Design")
  of the gradient cast to bf16: factored second moment (row and column means of g^2 + eps1, decayed by beta2_t = 1 - t^decay) for
  matrices, an unfactored one for vectors; update u = g / sqrt(v) clipped to RMS <= d; a running mean
  m of the clipped u, bias-corrected as Adam does; w -= lr * m_hat. Written from Shazeer and Stern's
  published algorithm (Adafactor, 2018), with the first moment the pages add.
"""
from __future__ import annotations

import math

import numpy as np
import torch

PARAMS_PER_BLOCK = ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down")
GLOBAL_PARAMS = ("embed", "final_norm", "pool_query", "pool_wk", "pool_wv")


def _t(a):
    return torch.tensor(np.asarray(a, dtype=np.float64), dtype=torch.float64, requires_grad=True)


def parameters(weights):
    """The float64 leaf tensors of a ``synth.Weights`` (matrices hold the bf16 values exactly)."""
    f = weights.f32
    p = {"embed": _t(f["embed"]), "final_norm": _t(f["final_norm"]), "pool_query": _t(f["pool_query"]),
         "pool_wk": _t(f["pool_wk"]), "pool_wv": _t(f["pool_wv"])}
    for name in PARAMS_PER_BLOCK:
        p[name] = [_t(x) for x in f[name]]
    return p


def _rmsnorm(x, g, eps):
    return x / torch.sqrt((x * x).mean(dim=1, keepdim=True) + eps) * g


def _rope(v, pos, heads, base):
    """1-axis rotary on [T x heads*64]: pair j of every head turns by pos * base^(-2j/64)."""
    T = v.shape[0]
    d = v.shape[1] // heads
    j = torch.arange(d // 2, dtype=torch.float64)
    phi = pos[:, None] * torch.pow(torch.tensor(base, dtype=torch.float64), -2.0 * j / d)[None, :]
    c, s = torch.cos(phi)[:, None, :], torch.sin(phi)[:, None, :]
    x = v.reshape(T, heads, d // 2, 2)
    x0, x1 = x[..., 0], x[..., 1]
    return torch.stack((x0 * c - x1 * s, x0 * s + x1 * c), dim=-1).reshape(T, heads * d)


def text_forward(p, geometry, data, offsets):
    """Pooled rows [count x D] (float64 torch) of a byte tape; items keep their first `context` bytes."""
    g = geometry
    D, H, N, eps = g["hidden"], g["heads"], g["depth"], g["rms_epsilon"]
    d = D // H
    off = np.asarray(offsets, dtype=np.int64)
    count = len(off) - 1
    lens = [min(int(off[i + 1] - off[i]), g["context"]) for i in range(count)]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    ids = np.concatenate([np.asarray(data[off[i]:off[i] + lens[i]], dtype=np.int64) for i in range(count)]) \
        if count else np.zeros(0, np.int64)
    pos = torch.tensor(np.concatenate([np.arange(n) for n in lens]) if count else np.zeros(0), dtype=torch.float64)
    x = p["embed"][torch.as_tensor(ids)]
    for l in range(N):
        h = _rmsnorm(x, p["attn_norm"][l], eps)
        qkv = h @ p["w_qkv"][l]
        q, k, v = qkv[:, :D], qkv[:, D:2 * D], qkv[:, 2 * D:]
        q, k = _rope(q, pos, H, g["rope_base"]), _rope(k, pos, H, g["rope_base"])
        outs = []
        for i in range(count):
            a, b = cu[i], cu[i + 1]
            if b == a:
                continue
            qi = q[a:b].reshape(b - a, H, d).transpose(0, 1)
            ki = k[a:b].reshape(b - a, H, d).transpose(0, 1)
            vi = v[a:b].reshape(b - a, H, d).transpose(0, 1)
            att = torch.softmax(qi @ ki.transpose(1, 2) / math.sqrt(d), dim=-1)
            outs.append((att @ vi).transpose(0, 1).reshape(b - a, D))
        o = torch.cat(outs) if outs else x[:0]
        x = x + o @ p["w_o"][l]
        h2 = _rmsnorm(x, p["mlp_norm"][l], eps)
        gate, up = h2 @ p["w_gate"][l], h2 @ p["w_up"][l]
        x = x + (gate * torch.sigmoid(gate) * up) @ p["w_down"][l]
    xf = _rmsnorm(x, p["final_norm"], eps)
    kk, vv = xf @ p["pool_wk"], xf @ p["pool_wv"]
    rows = []
    for i in range(count):
        a, b = cu[i], cu[i + 1]
        if b == a:
            rows.append(torch.zeros(D, dtype=torch.float64))
            continue
        ki = kk[a:b].reshape(b - a, H, d)
        vi = vv[a:b].reshape(b - a, H, d)
        s = (ki * p["pool_query"].reshape(1, H, d)).sum(-1) / math.sqrt(d)  # [L x H]
        w = torch.softmax(s, dim=0)
        rows.append((w[:, :, None] * vi).sum(0).reshape(D))
    return torch.stack(rows) if rows else torch.zeros((0, D), dtype=torch.float64)


def text_backward(weights, data, offsets, d_pooled):
    """(pooled, gradients): gradients of sum(pooled * d_pooled) for every parameter, float64 numpy,
    keyed like the weights (per-block entries are lists)."""
    p = parameters(weights)
    pooled = text_forward(p, weights.geometry, data, offsets)
    (pooled * torch.as_tensor(np.asarray(d_pooled, dtype=np.float64))).sum().backward()
    grads = {}
    for name, v in p.items():
        if isinstance(v, list):
            grads[name] = [x.grad.numpy().copy() if x.grad is not None else np.zeros(x.shape) for x in v]
        else:
            grads[name] = v.grad.numpy().copy() if v.grad is not None else np.zeros(v.shape)
    return pooled.detach().numpy(), grads


# ---------------------------------------------------------------------------------------- Adafactor

class AdafactorState:
    """Per-tensor optimizer state: row and column second moments (matrices) or a full one (vectors), and
    the first moment."""

    def __init__(self, shape):
        self.shape = tuple(shape)
        if len(shape) == 2:
            self.r = np.zeros(shape[0])
            self.c = np.zeros(shape[1])
        else:
            self.v = np.zeros(shape)
        self.m = np.zeros(shape)


def bf16_round(a):
    """Float32 values rounded to bfloat16 (nearest even) by the library cast, back in float64."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def adafactor(w, g, state, lr, step, beta1=0.9, decay=-0.8, eps1=1e-30, clip=1.0, grad_bf16=True):
    """One update of tensor w (float64 values) with gradient g at step `step` (counted from 1); returns
    the new values and updates `state` in place. With ``grad_bf16`` the float32 gradient is cast to bf16
    first ("Precision by Design": gradients accumulate in float32 and are cast to BF16 for the step)."""
    w = np.asarray(w, dtype=np.float64)
    g = bf16_round(g) if grad_bf16 else np.asarray(g, dtype=np.float64)
    beta2 = 1.0 - step ** decay
    sq = g * g + eps1
    if g.ndim == 2:
        state.r = beta2 * state.r + (1.0 - beta2) * sq.mean(axis=1)
        state.c = beta2 * state.c + (1.0 - beta2) * sq.mean(axis=0)
        v = np.outer(state.r, state.c) / state.r.mean()
    else:
        state.v = beta2 * state.v + (1.0 - beta2) * sq
        v = state.v
    u = g / np.sqrt(v)
    u = u / max(1.0, math.sqrt(float(np.mean(u * u))) / clip)
    state.m = beta1 * state.m + (1.0 - beta1) * u
    m_hat = state.m / (1.0 - beta1 ** step)
    return w - lr * m_hat
