"""Training step of the HIP path (backward pass and Adafactor) against the float64 oracle, through the C ABI.

Bars (derived in the design notes): every parameter's gradient within cosine >= 0.995 of the float64
oracle and max |difference| <= 5e-2 of its largest entry (the replayed forward and every backward
intermediate are stored in bf16, ~2^-9 relative each, over a dozen chained products); the Adafactor update
of the GPU's own gradients within one bf16 step of the oracle's update of the same gradients; after the
step, the model's encodes equal the oracle's forward with the updated masters (the pooled-row bar).
"""
import numpy as np
import pytest

import oracle
from multimodal_embeddings_amd import configs, synth
from oracle import train as TR
from tests.gpu_util import COS_MIN, device_bytes, row_cos, say

pytestmark = pytest.mark.gpu

GRAD_COS = 0.995
GRAD_REL = 5e-2


@pytest.fixture(scope="module")
def ube():
    import multimodal_embeddings_amd as m
    return m


def _setup(ube, name="tiny", count=None, seed=1):
    g = configs.geometry(name)
    w = synth.make_weights(g, gain_jitter=0.2)
    batch = synth.workload_inputs(name) if count is None else synth.text_batch(count, 16, 200, 0, 256, seed=seed)
    model = ube.Model(w, 0)
    trainer = ube.Trainer(model, w)
    arena = ube.Arena(0)
    return g, w, batch, model, trainer, arena


def _grads_by_name(trainer):
    out = {}
    for name, layer, master, grad in trainer.tensors():
        out[(name, layer)] = (master, grad.double().cpu().numpy())
    return out


def _compare_grads(label, got, want_grads, depth):
    worst = (1.0, 0.0)
    for name in TR.GLOBAL_PARAMS + TR.PARAMS_PER_BLOCK:
        refs = want_grads[name] if isinstance(want_grads[name], list) else [want_grads[name]]
        for layer, ref in enumerate(refs):
            g = got[(name, layer)][1].reshape(ref.shape)
            scale = np.abs(ref).max()
            cos = float((g * ref).sum() / (np.linalg.norm(g) * np.linalg.norm(ref))) if scale > 0 else 1.0
            err = np.abs(g - ref).max() / scale if scale > 0 else np.abs(g).max()
            say(f"[{label}] d{name}[{layer}] {ref.shape}: cos {cos:.6f}, max |diff| {err:.2e} of max")
            assert cos >= GRAD_COS and err <= GRAD_REL, (label, name, layer, cos, err)
            worst = (min(worst[0], cos), max(worst[1], err))
    return worst


@pytest.mark.parametrize("name,count", [("tiny", None), ("tiny", 5)])
def test_backward_matches_oracle(ube, name, count):
    g, w, batch, model, trainer, arena = _setup(ube, name, count)
    rng = np.random.default_rng(7)
    d_pooled = rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)
    say(f"[{name}] items {batch.count}, bytes {int(batch.offsets[-1])}")
    trainer.backward(arena, device_bytes(batch.data), batch.offsets, device_bytes(d_pooled))
    import torch
    torch.cuda.synchronize()
    _, want = TR.text_backward(w, batch.data, batch.offsets, d_pooled)
    worst = _compare_grads(name, _grads_by_name(trainer), want, g["depth"])
    say(f"[{name}] worst gradient cosine {worst[0]:.6f}, worst max |diff| {worst[1]:.2e}")


def test_adafactor_step_and_refreshed_forward(ube):
    import torch
    g, w, batch, model, trainer, arena = _setup(ube, "tiny")
    rng = np.random.default_rng(8)
    d_pooled = rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)
    data = device_bytes(batch.data)
    trainer.backward(arena, data, batch.offsets, device_bytes(d_pooled))
    torch.cuda.synchronize()
    before = {(n, l): (m.float().cpu().numpy().astype(np.float64), gr.double().cpu().numpy())
              for n, l, m, gr in trainer.tensors()}
    lr = 1e-3
    trainer.step(lr)
    torch.cuda.synchronize()
    after = {(n, l): m.float().cpu().numpy().astype(np.float64) for n, l, m, _ in trainer.tensors()}
    worst = 0.0
    for key, (w0, gr) in before.items():
        st = TR.AdafactorState(w0.shape)
        want = TR.adafactor(w0, gr, st, lr, 1)
        got = after[key]
        bf16 = key[0] not in ("attn_norm", "mlp_norm", "final_norm")
        if bf16:  # masters are bf16: compare against the oracle's update rounded the same way
            want = synth.bf16_bits_to_f32(synth.to_bf16_bits(want.astype(np.float32))).astype(np.float64)
            ulp = np.abs(want) * 2.0 ** -7 + 1e-30
            steps = np.abs(got - want) / ulp
            worst = max(worst, float(steps.max()))
            assert steps.max() <= 1.0, (key, steps.max())
        else:
            assert np.allclose(got, want, rtol=1e-5, atol=1e-7), key
    say(f"[adafactor] step 1 of every tensor: worst bf16 difference {worst:.2f} steps")
    # the model now encodes with the updated masters
    upd = synth.make_weights(g, gain_jitter=0.2)
    for n, l, m, _ in trainer.tensors():
        vals = m.float().cpu().numpy()
        if n in ("attn_norm", "mlp_norm"):
            upd.f32[n][l] = vals.astype(np.float32)
        elif n == "final_norm":
            upd.f32[n] = vals.astype(np.float32)
        elif n in TR.PARAMS_PER_BLOCK:
            synth.set_matrix(upd, n, vals, l)
        else:
            synth.set_matrix(upd, n, vals)
    rows, _ = ube.text_encode(model, arena, data, batch.offsets)
    got = rows.tensor().double().cpu().numpy()
    want, _ = oracle.encode_text(upd, batch.data, batch.offsets)
    cos = row_cos(got, want)
    err = np.abs(got - want).max()
    say(f"[refreshed forward] min cos {cos.min():.6f}, max |diff| {err:.2e}")
    assert cos.min() >= COS_MIN and err <= 2e-2
