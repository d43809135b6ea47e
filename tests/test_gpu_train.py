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


def _setup(ube, name="tiny", count=None, seed=1, recompute=False):
    g = configs.geometry(name)
    w = synth.make_weights(g, gain_jitter=0.2)
    batch = synth.workload_inputs(name) if count is None else synth.text_batch(count, 16, 200, 0, 256, seed=seed)
    model = ube.Model(w, 0)
    trainer = ube.Trainer(model, w, activation_recomputation=recompute)
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


@pytest.mark.parametrize("name,count,recompute", [("tiny", None, False), ("tiny", 5, False), ("tiny", None, True)])
def test_backward_matches_oracle(ube, name, count, recompute):
    g, w, batch, model, trainer, arena = _setup(ube, name, count, recompute=recompute)
    rng = np.random.default_rng(7)
    d_pooled = rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)
    say(f"[{name}] items {batch.count}, bytes {int(batch.offsets[-1])}")
    trainer.backward(arena, device_bytes(batch.data), batch.offsets, device_bytes(d_pooled))
    import torch
    torch.cuda.synchronize()
    _, want = TR.text_backward(w, batch.data, batch.offsets, d_pooled)
    worst = _compare_grads(name, _grads_by_name(trainer), want, g["depth"])
    say(f"[{name}] worst gradient cosine {worst[0]:.6f}, worst max |diff| {worst[1]:.2e}")


def test_backward_edge_cases(ube):
    """Empty items among others (their pooled rows are zero and pass no gradient), an item cut at the
    context (1100 bytes, the first 1024 kept), and an empty tape (every gradient zero)."""
    import torch
    g, w, _, model, trainer, arena = _setup(ube, "tiny")
    rng = np.random.default_rng(15)
    lengths = [0, 5, 1100, 0, 37]
    data = rng.integers(0, 256, size=sum(lengths), dtype=np.int64).astype(np.uint8)
    offsets = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint64)
    d_pooled = rng.standard_normal((len(lengths), g["hidden"])).astype(np.float32)
    truncated, tokens = trainer.backward(arena, device_bytes(data), offsets, device_bytes(d_pooled))
    torch.cuda.synchronize()
    assert (truncated, tokens) == (1, 5 + 1024 + 37)
    _, want = TR.text_backward(w, data, offsets, d_pooled)
    worst = _compare_grads("edges", _grads_by_name(trainer), want, g["depth"])
    say(f"[edges] worst gradient cosine {worst[0]:.6f}, worst max |diff| {worst[1]:.2e}")
    trainer.backward(arena, device_bytes(np.zeros(1, np.uint8)), np.zeros(1, np.uint64), None)
    torch.cuda.synchronize()
    assert all(float(gr.abs().max()) == 0.0 for _, _, _, gr in trainer.tensors())


def test_tensor_views_keep_the_trainer_alive(ube):
    import gc
    import torch
    g, w, batch, model, trainer, arena = _setup(ube)
    views = trainer.tensors()
    assert all(m.device == torch.device("cuda:0") for _, _, m, _ in views)
    first = views[0][2].float().cpu().clone()
    with pytest.raises(RuntimeError):
        trainer.close()  # views alive: the memory must not be freed under them
    del trainer
    gc.collect()
    # the trainer object is gone from this scope, but its memory is not: the views hold it
    np.testing.assert_array_equal(views[0][2].float().cpu().numpy(), first.numpy())
    del views
    gc.collect()
    t2 = ube.Trainer(model, w)
    v2 = t2.tensors()
    del v2
    gc.collect()
    t2.close()  # no views left: closes
    arena.close()


def test_trainer_refuses_unsupported_geometry(ube):
    """A model the encoder runs (ffn 320, a multiple of 64) but whose activation-gradient products the
    trainer's 128-column tiles cannot cover: the trainer reports unsupported instead of failing later."""
    g = dict(configs.geometry("tiny"))
    g["ffn"] = 320
    w = synth.make_weights(g)
    model = ube.Model(w, 0)
    with pytest.raises(ube.UbeError) as e:
        ube.Trainer(model, w)
    assert e.value.status == "unsupported", e.value


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
            # one bf16 step of the result, plus the fp32 arithmetic of w - lr m_hat (a few fp32 ulps of the
            # operands: where w and the update nearly cancel, the result is far below them)
            upd = np.abs(want - w0)
            want = synth.bf16_bits_to_f32(synth.to_bf16_bits(want.astype(np.float32))).astype(np.float64)
            ulp = np.abs(want) * 2.0 ** -7 + (np.abs(w0) + upd) * 2.0 ** -20 + 1e-30
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


def test_forward_then_backward(ube):
    """The training forward returns the encode's rows bit for bit, and a backward over its kept activations
    equals the self-contained backward bit for bit; after a step the kept activations are refused."""
    import torch
    g, w, batch, model, trainer, arena = _setup(ube, "tiny", 6, seed=4)
    data = device_bytes(batch.data)
    d = torch.from_numpy(np.random.default_rng(11).standard_normal((batch.count, g["hidden"])).astype(np.float32)).cuda()
    rows, (_, tokens) = trainer.forward(arena, data, batch.offsets)
    got = rows.tensor()
    enc, _ = ube.text_encode(model, arena, data, batch.offsets)
    assert tokens == int(np.diff(batch.offsets).sum()) and torch.equal(got, enc.tensor())
    trainer.backward(None, None, None, d, after_forward=True)
    torch.cuda.synchronize()
    kept = [gr.clone() for _, _, _, gr in trainer.tensors()]
    trainer.backward(arena, data, batch.offsets, d)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(kept, [gr for _, _, _, gr in trainer.tensors()]))
    # the self-contained backward leaves its own forward kept: a second pass over it agrees too
    trainer.backward(None, None, None, d, after_forward=True)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(kept, [gr for _, _, _, gr in trainer.tensors()]))
    trainer.step(1e-3)
    with pytest.raises(ube.UbeError):
        trainer.backward(None, None, None, d, after_forward=True)


def test_three_adafactor_steps_track_the_oracle(ube):
    """Three steps in a row: after each, every master equals the oracle's Adafactor run over the same
    sequence of GPU gradients (its own state carried from step to step: the decayed factored second
    moment, beta2_t = 1 - t^-0.8, the first moment and its bias correction), within one bf16 step plus
    the fp32 rounding of the update at the operands' scale."""
    import torch
    g, w, batch, model, trainer, arena = _setup(ube, "tiny")
    data = device_bytes(batch.data)
    rng = np.random.default_rng(21)
    states, masters = {}, {}
    for n, l, m, _ in trainer.tensors():
        masters[(n, l)] = m.float().cpu().numpy().astype(np.float64)
        states[(n, l)] = TR.AdafactorState(m.shape)
    lr = 1e-3
    worst = 0.0
    for step in (1, 2, 3):
        d_pooled = rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)
        trainer.backward(arena, data, batch.offsets, device_bytes(d_pooled))
        torch.cuda.synchronize()
        grads = {(n, l): gr.double().cpu().numpy() for n, l, _, gr in trainer.tensors()}
        trainer.step(lr)
        torch.cuda.synchronize()
        for n, l, m, _ in trainer.tensors():
            key = (n, l)
            w0 = masters[key]
            want = TR.adafactor(w0, grads[key], states[key], lr, step)
            got = m.float().cpu().numpy().astype(np.float64)
            if n in ("attn_norm", "mlp_norm", "final_norm"):
                assert np.allclose(got, want, rtol=1e-5, atol=1e-7), (key, step)
            else:
                upd = np.abs(want - w0)
                want = synth.bf16_bits_to_f32(synth.to_bf16_bits(want.astype(np.float32))).astype(np.float64)
                bar = np.abs(want) * 2.0 ** -7 + (np.abs(w0) + upd) * 2.0 ** -20 + 1e-30
                steps = float((np.abs(got - want) / bar).max())
                worst = max(worst, steps)
                assert steps <= 1.0, (key, step, steps)
            masters[key] = got  # the next step starts from the GPU's own masters
    say(f"[adafactor x3] worst bf16 difference over three steps {worst:.2f} steps")


def test_training_lowers_the_contrastive_loss(ube):
    """End to end on 16 rows of 256 bytes at depth 12: forward, Matryoshka sigmoid loss over pairs
    (2k, 2k + 1), backward and Adafactor step (learning rate 2e-4), five times; the loss of the same batch
    falls after the first step and ends below where it started."""
    import torch
    g = configs.geometry("text512")
    w = synth.make_weights(g)
    batch = synth.text_batch(16, 256, 257, 0, 256, seed=14)
    model, arena, arena2 = ube.Model(w, 0), ube.Arena(0), ube.Arena(0)
    trainer = ube.Trainer(model, w)
    data = device_bytes(batch.data)
    n = batch.count
    pairs = synth.Edges.from_lists([[i ^ 1] for i in range(n)])
    widths = (64, 128, 256, 512)
    scalars = torch.zeros(3 + len(widths), device="cuda")
    gemb = torch.zeros((n, g["hidden"]), device="cuda")
    losses = []
    for _ in range(5):
        rows, _ = trainer.forward(arena, data, batch.offsets)
        emb = rows.tensor().to(torch.bfloat16)
        ube.contrastive(arena2, emb, scalars, widths=widths, attract=(pairs.offsets, pairs.ids, None), gradient=gemb)
        torch.cuda.synchronize()
        losses.append(float(scalars[0]))
        trainer.backward(None, None, None, gemb, after_forward=True)
        trainer.step(2e-4)
        torch.cuda.synchronize()
    say(f"[end to end] contrastive loss over five steps: {', '.join(f'{x:.4f}' for x in losses)}")
    # a small step along Adafactor's (sign-like, clipped) update lowers the loss to first order
    assert all(np.isfinite(losses)) and losses[1] < losses[0] and losses[-1] < losses[0]


@pytest.mark.parametrize("recompute", [False, True])
def test_depth12_backward_matches_oracle(ube, recompute):
    """The depth-12, hidden-512 encoder on a few ragged rows (cosine and max-difference bars as above), with
    every activation kept and with each block's attention half replayed from its fp32 input."""
    import torch
    g = configs.geometry("text512")
    w = synth.make_weights(g, gain_jitter=0.2)
    batch = synth.text_batch(4, 100, 400, 0, 256, seed=3)
    model, arena = ube.Model(w, 0), ube.Arena(0)
    trainer = ube.Trainer(model, w, activation_recomputation=recompute)
    rng = np.random.default_rng(9)
    d_pooled = rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)
    trainer.backward(arena, device_bytes(batch.data), batch.offsets, device_bytes(d_pooled))
    torch.cuda.synchronize()
    _, want = TR.text_backward(w, batch.data, batch.offsets, d_pooled)
    worst = _compare_grads("text512", _grads_by_name(trainer), want, g["depth"])
    say(f"[text512] worst gradient cosine {worst[0]:.6f}, worst max |diff| {worst[1]:.2e}")


@pytest.mark.parametrize("name", ["text768_shallow", "text1024_shallow"])
def test_wide_backward_matches_oracle(ube, name):
    """Hidden 768 (12 heads) and 1024 (16 heads), depth 2, a few ragged rows: the wider pool and norm paths
    and heads beyond one group of 8 (cosine and max-difference bars as above)."""
    import torch
    g = configs.geometry(name)
    w = synth.make_weights(g, gain_jitter=0.2)
    batch = synth.text_batch(3, 60, 300, 0, 256, seed=12)
    model, arena = ube.Model(w, 0), ube.Arena(0)
    trainer = ube.Trainer(model, w)
    rng = np.random.default_rng(13)
    d_pooled = rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)
    trainer.backward(arena, device_bytes(batch.data), batch.offsets, device_bytes(d_pooled))
    torch.cuda.synchronize()
    _, want = TR.text_backward(w, batch.data, batch.offsets, d_pooled)
    worst = _compare_grads(name, _grads_by_name(trainer), want, g["depth"])
    say(f"[{name}] worst gradient cosine {worst[0]:.6f}, worst max |diff| {worst[1]:.2e}")


def test_full_size_linearity_and_zero(ube):
    """The training step's full batch (64 rows x 1024 bytes, depth 12): gradients are linear in the upstream
    gradient (the backward of d1 + d2 equals the sum of the two) and vanish for a zero upstream gradient."""
    import torch
    g = configs.geometry("text512")
    w = synth.make_weights(g)
    batch = synth.workload_inputs("train")
    model, arena = ube.Model(w, 0), ube.Arena(0)
    trainer = ube.Trainer(model, w)
    data = device_bytes(batch.data)
    rng = np.random.default_rng(10)
    d1 = torch.from_numpy(rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)).cuda()
    d2 = torch.from_numpy(rng.standard_normal((batch.count, g["hidden"])).astype(np.float32)).cuda()

    def grads(d):
        trainer.backward(arena, data, batch.offsets, d)
        torch.cuda.synchronize()
        return [gr.double().clone() for _, _, _, gr in trainer.tensors()]

    a, b, ab = grads(d1), grads(d2), grads(d1 + d2)
    worst = 0.0
    for x, y, z in zip(a, b, ab):
        s = x + y
        scale = s.abs().max().item()
        if scale > 0:
            worst = max(worst, ((z - s).abs().max() / scale).item())
    say(f"[full size] linearity: worst max |g(d1 + d2) - g(d1) - g(d2)| = {worst:.2e} of max")
    assert worst <= 2e-2
    zero = grads(torch.zeros_like(d1))
    assert all(float(x.abs().max()) == 0.0 for x in zero)
