"""Pins of the training-step oracle (CPU only): the float64 torch forward against the pinned C oracle,
autograd gradients against central finite differences, and Adafactor against hand-derived updates."""
import math

import numpy as np
import pytest

import oracle
from multimodal_embeddings_amd import configs, synth
from oracle import train as TR


def _tiny_case(seed=1):
    g = configs.geometry("tiny")
    w = synth.make_weights(g, gain_jitter=0.2)
    batch = synth.text_batch(3, 5, 10, 0, 256, seed=seed)
    return g, w, batch


def test_torch_forward_equals_c_oracle():
    g, w, _ = _tiny_case()
    batch = synth.workload_inputs("tiny")
    want, _ = oracle.encode_text(w, batch.data, batch.offsets)
    got = TR.text_forward(TR.parameters(w), w.geometry, batch.data, batch.offsets).detach().numpy()
    assert np.allclose(got, want, rtol=1e-10, atol=1e-13)


def test_backward_matches_finite_differences():
    g, w, batch = _tiny_case()
    rng = np.random.default_rng(5)
    d_pooled = rng.standard_normal((batch.count, g["hidden"]))
    _, grads = TR.text_backward(w, batch.data, batch.offsets, d_pooled)
    p = TR.parameters(w)

    def loss():
        with np_no_grad():
            return float((TR.text_forward(p, w.geometry, batch.data, batch.offsets).detach().numpy() * d_pooled).sum())

    checked = 0
    for name in TR.GLOBAL_PARAMS + TR.PARAMS_PER_BLOCK:
        tensors = p[name] if isinstance(p[name], list) else [p[name]]
        refs = grads[name] if isinstance(grads[name], list) else [grads[name]]
        for t, ref in zip(tensors, refs):
            flat = t.data.view(-1)
            if name == "embed":  # rows the tape uses
                used = np.unique(batch.data)
                picks = [int(used[0]) * t.shape[1] + 3, int(used[-1]) * t.shape[1] + 17]
            else:
                picks = rng.choice(flat.numel(), size=3, replace=False).tolist()
            for idx in picks:
                h = 1e-6 * max(1.0, abs(float(flat[idx])))
                old = float(flat[idx])
                flat[idx] = old + h
                lp = loss()
                flat[idx] = old - h
                lm = loss()
                flat[idx] = old
                fd = (lp - lm) / (2 * h)
                got = float(ref.reshape(-1)[idx])
                assert got == pytest.approx(fd, rel=2e-5, abs=1e-9), (name, idx, got, fd)
                checked += 1
    assert checked > 40


class np_no_grad:
    def __enter__(self):
        import torch
        self._g = torch.no_grad()
        self._g.__enter__()

    def __exit__(self, *a):
        self._g.__exit__(*a)


def test_adafactor_first_step_is_sign_descent():
    rng = np.random.default_rng(0)
    # vector: v = g^2, u = sign(g), no clipping at RMS 1, bias-corrected first moment = u
    w, g = rng.standard_normal(7), rng.standard_normal(7)
    st = TR.AdafactorState(w.shape)
    assert np.allclose(TR.adafactor(w, g, st, 0.01, 1, grad_bf16=False), w - 0.01 * np.sign(g), rtol=0, atol=1e-15)
    # matrix with rank-one g^2: the factored second moment is exact
    a, b = rng.standard_normal(5), rng.standard_normal(4)
    G = np.outer(a, b)
    W = rng.standard_normal((5, 4))
    st = TR.AdafactorState(W.shape)
    assert np.allclose(TR.adafactor(W, G, st, 0.02, 1, grad_bf16=False), W - 0.02 * np.sign(G), rtol=0, atol=1e-12)
    assert np.allclose(st.r, (G * G).mean(1) + 1e-30) and np.allclose(st.c, (G * G).mean(0) + 1e-30)


def test_adafactor_second_step_clipping_and_bias_correction():
    n = 6
    w = np.zeros(n)
    st = TR.AdafactorState((n,))
    w1 = TR.adafactor(w, np.full(n, 1e-10), st, 0.5, 1, grad_bf16=False)
    assert np.allclose(w1, -0.5)
    w2 = TR.adafactor(w1, np.ones(n), st, 0.5, 2, grad_bf16=False)
    beta2 = 1 - 2 ** -0.8
    u = 1 / math.sqrt(beta2 * (1e-20 + 1e-30) + (1 - beta2) * (1 + 1e-30))
    assert u > 1.3  # clipped back to RMS 1
    m2 = 0.9 * 0.1 + 0.1 * 1.0
    assert np.allclose(w2, w1 - 0.5 * m2 / (1 - 0.81), rtol=1e-12)


def test_adafactor_is_gradient_scale_free():
    rng = np.random.default_rng(2)
    W, G1, G2 = rng.standard_normal((6, 3)), rng.standard_normal((6, 3)), rng.standard_normal((6, 3))
    s1, s2 = TR.AdafactorState(W.shape), TR.AdafactorState(W.shape)
    a = TR.adafactor(TR.adafactor(W, G1, s1, 0.1, 1, grad_bf16=False), G2, s1, 0.1, 2, grad_bf16=False)
    b = TR.adafactor(TR.adafactor(W, 1e3 * G1, s2, 0.1, 1, grad_bf16=False), 1e3 * G2, s2, 0.1, 2, grad_bf16=False)
    assert np.allclose(a, b, rtol=1e-9)


def test_adafactor_reads_the_gradient_at_bf16_precision():
    rng = np.random.default_rng(3)
    W = rng.standard_normal((5, 7))
    G = TR.bf16_round(rng.standard_normal((5, 7)))  # bf16 values
    a = TR.adafactor(W, G, TR.AdafactorState(W.shape), 0.05, 1)
    # a relative change of 2^-10 is below half a bf16 step: the cast takes it back to G
    b = TR.adafactor(W, G * (1 + 2.0 ** -10), TR.AdafactorState(W.shape), 0.05, 1)
    assert np.array_equal(a, b)
    # one of 2^-7 is a whole step: the update changes, and equals the update of the rounded gradient
    G2 = G * (1 + 2.0 ** -7)
    c = TR.adafactor(W, G2, TR.AdafactorState(W.shape), 0.05, 1)
    assert not np.array_equal(a, c)
    d = TR.adafactor(W, TR.bf16_round(G2), TR.AdafactorState(W.shape), 0.05, 1, grad_bf16=False)
    assert np.array_equal(c, d)
    # the cast is the nearest-even rounding to 8 significant bits
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -9, -(1 + 2.0 ** -7 + 2.0 ** -9)])
    assert np.array_equal(TR.bf16_round(x), [1.0, 1 + 2.0 ** -6, 1.0, -(1 + 2.0 ** -7)])
