"""Per-token outputs (final-norm states, token-head unit vectors) and the hard
MaxSim scorer of the HIP path against the CPU oracle, through the C ABI.

Bars: states and token vectors per row cosine >= 0.999 and max |difference|
<= 2e-2 against the float64 oracle (the pooled-row bar); rows-tape metadata
and offsets bit-exact; embeddings unchanged by the extra surfaces (bit-exact).
MaxSim of the GPU's own bf16 token vectors against the oracle's MaxSim of the
same values: |difference| <= 1e-4 (fp32 sums of 128 bf16 products against
float64); end to end against the oracle's own token vectors: <= 2e-2.
"""
import numpy as np
import pytest

import oracle
from multimodal_embeddings_amd import configs, synth
from tests.gpu_util import COS_MIN, ABS_MAX, device_bytes, row_cos, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ube():
    import multimodal_embeddings_amd as m
    return m


_MODELS = {}


def _model(ube, name, **kw):
    key = (name, tuple(sorted(kw.items())))
    if key not in _MODELS:
        w = synth.make_weights(configs.geometry(name), **kw)
        _MODELS[key] = (w, ube.Model(w, 0), ube.Arena(0))
    return _MODELS[key]


# Per-token rows are not averaged over an item as the pooled rows are: besides the pooled-row bar's
# absolute part, each value may carry one bf16 step of its own magnitude (the blocks store every activation
# in bf16, and a single token's state keeps the rounding that pooling averages away).
TOKEN_REL = 2.0 ** -7


def _check_rows(got, want, label):
    got = np.asarray(got, np.float64)
    cos = row_cos(got, want)
    diff = np.abs(got - want)
    err = diff.max() if want.size else 0.0
    ratio = (diff / (ABS_MAX + TOKEN_REL * np.abs(want))).max() if want.size else 0.0
    say(f"[{label}] rows {len(want)}: min cos {cos.min() if len(cos) else 1:.6f}, max |diff| {err:.3e}, "
        f"worst |diff| / bar {ratio:.3f}")
    assert cos.min() >= COS_MIN, (label, cos.min())
    assert ratio <= 1.0, (label, err, ratio)


def _oracle_token_outputs(w, data, offsets):
    g = w.geometry
    lengths, cu, stats = oracle.tape_plan(offsets, g["context"])
    x0, pos = oracle.embed_text(data, offsets, lengths, cu, w.f32["embed"])
    _, xf = oracle.forward_states(w, x0, pos, cu)
    return xf, oracle.token_vectors(xf, w.f32["token_head"]), cu, stats


@pytest.mark.parametrize("scalar", ["f32", "bf16"])
def test_tiny_states_and_token_vectors_match_oracle(ube, scalar):
    w, model, arena = _model(ube, "tiny", gain_jitter=0.2)
    batch = synth.workload_inputs("tiny")
    assert model.describe()["token_width"] == 128
    emb, states, vecs, stats = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets,
                                               outputs_scalar=scalar,
                                               outputs=("embeddings", "states", "token_vectors"))
    xf, tv, cu, ostats = _oracle_token_outputs(w, batch.data, batch.offsets)
    assert stats == ostats
    T, D = int(cu[-1]), w.geometry["hidden"]
    item = 4 if scalar == "f32" else 2
    assert (states.count, states.rows, states.columns, states.stride, states.scalar) == (8, T, D, D * item, scalar)
    assert (vecs.count, vecs.rows, vecs.columns, vecs.stride, vecs.scalar) == (8, T, 128, 128 * item, scalar)
    np.testing.assert_array_equal(states.offsets(), cu.astype(np.uint64))
    np.testing.assert_array_equal(vecs.offsets(), cu.astype(np.uint64))
    gs = states.tensor().double().cpu().numpy()
    gv = vecs.tensor().double().cpu().numpy()
    _check_rows(gs, xf, f"tiny states {scalar}")
    _check_rows(gv, tv, f"tiny token vectors {scalar}")
    norms = np.linalg.norm(gv, axis=1)
    assert np.abs(norms - 1).max() <= (1e-5 if scalar == "f32" else 8e-3), np.abs(norms - 1).max()
    # the extra surfaces leave the pooled rows untouched (bit-exact)
    plain, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets, outputs_scalar=scalar)
    a = plain.tensor().float().cpu().numpy()
    _, _, _, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets, outputs_scalar=scalar,
                                 outputs=("states",))
    emb2, _, _, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets, outputs_scalar=scalar,
                                    outputs=("embeddings", "token_vectors"))
    np.testing.assert_array_equal(emb2.tensor().float().cpu().numpy(), a)


def test_surfaces_left_out_are_empty_and_missing_head_is_unsupported(ube):
    w, model, arena = _model(ube, "tiny")
    batch = synth.workload_inputs("tiny")
    emb, states, vecs, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets,
                                           outputs=("states",))
    assert emb is None and vecs is None and states.rows == int(batch.offsets[-1])
    # a model without the token head
    g = dict(configs.geometry("tiny"))
    g["token_width"] = 0
    w0 = synth.make_weights(g)
    m0 = ube.Model(w0, 0)
    with pytest.raises(ube.UbeError, match="unsupported"):
        ube.text_encode(m0, arena, device_bytes(batch.data), batch.offsets, outputs=("token_vectors",))
    assert m0.describe()["token_width"] == 0
    m0.close()


def test_ragged_states_and_token_vectors_sampled(ube):
    w, model, arena = _model(ube, "text512")
    batch = synth.workload_inputs("ragged")
    _, states, vecs, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets,
                                         outputs=("states", "token_vectors"))
    off = states.offsets()
    gs, gv = states.tensor().double().cpu().numpy(), vecs.tensor().double().cpu().numpy()
    rows = [0, 17, 63]
    sub = synth.subset(batch, rows)
    xf, tv, cu, _ = _oracle_token_outputs(w, sub.data, sub.offsets)
    for k, i in enumerate(rows):
        a, b = int(off[i]), int(off[i + 1])
        _check_rows(gs[a:b], xf[cu[k]:cu[k + 1]], f"ragged states item {i}")
        _check_rows(gv[a:b], tv[cu[k]:cu[k + 1]], f"ragged token vectors item {i}")


def _maxsim_gpu(ube, q, d, prefix=0, span=0):
    import torch
    scores = torch.full((q.count, max(d.count, 1)), float("nan"), dtype=torch.float32, device="cuda:0")
    ube.maxsim(q, d, scores, prefix=prefix, span=span)
    return scores.cpu().numpy()[:, :d.count].astype(np.float64)


def test_maxsim_matches_oracle_on_the_same_vectors(ube):
    import torch
    w, model, arena = _model(ube, "tiny", gain_jitter=0.2)
    batch = synth.workload_inputs("tiny")
    _, _, vecs, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets, outputs_scalar="bf16",
                                    outputs=("token_vectors",))
    v = vecs.tensor().clone()
    off = torch.from_numpy(vecs.offsets().astype(np.int64)).to("cuda:0")
    tape = ube.rows_tape(v, off)
    host = v.double().cpu().numpy()
    ho = vecs.offsets()
    for prefix, span in ((0, 0), (0, 16), (5, 64), (70, 64)):
        got = _maxsim_gpu(ube, tape, tape, prefix, span)
        want = oracle.maxsim(host, ho, host, ho, prefix=prefix, span=span or 64)
        say(f"[maxsim prefix {prefix} span {span}] max |diff| {np.abs(got - want).max():.3e}")
        assert np.abs(got - want).max() <= 1e-4
    # items scored against themselves: every query row finds itself (<= 1 up to rounding)
    diag = np.diag(_maxsim_gpu(ube, tape, tape))
    assert np.all(np.abs(diag - 1) <= 1e-2)
    # end to end against the oracle's own token vectors
    _, tv, cu, _ = _oracle_token_outputs(w, batch.data, batch.offsets)
    e2e = oracle.maxsim(tv, cu, tv, cu)
    assert np.abs(_maxsim_gpu(ube, tape, tape) - e2e).max() <= ABS_MAX


def test_maxsim_empty_items_and_ragged_documents(ube):
    import torch
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((300, 128))
    rows /= np.linalg.norm(rows, axis=1, keepdims=True)
    bf = torch.from_numpy(rows.astype(np.float32)).to(torch.bfloat16)
    host = bf.double().numpy()
    v = bf.to("cuda:0")
    # queries: lengths 0, 1, 70 (two 64-row passes), 3; documents: 0, 33, 1, 100, 200 - 134 rows
    qo = np.array([0, 0, 1, 71, 74], np.uint64)
    do = np.array([74, 74, 107, 108, 208, 300], np.uint64)
    qt = ube.rows_tape(v, torch.from_numpy(qo.astype(np.int64)).to("cuda:0"))
    dt = ube.rows_tape(v, torch.from_numpy(do.astype(np.int64)).to("cuda:0"))
    for span in (0, 128):
        got = _maxsim_gpu(ube, qt, dt, 0, span)
        want = oracle.maxsim(host, qo, host, do, prefix=0, span=span or 64)
        assert np.abs(got - want).max() <= 1e-4, np.abs(got - want).max()
        assert np.all(got[0] == 0) and np.all(got[:, 0] == 0)  # empty query, empty document (reading)


def test_maxsim_refuses_bad_inputs(ube):
    import torch
    v = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda:0")
    off = torch.tensor([0, 8], dtype=torch.int64, device="cuda:0")
    t = ube.rows_tape(v, off)
    scores = torch.zeros((1, 1), dtype=torch.float32, device="cuda:0")
    with pytest.raises(ube.UbeError, match="unsupported"):
        ube.maxsim(t, t, scores)  # width 64
    f = ube.rows_tape(torch.zeros((8, 128), dtype=torch.float32, device="cuda:0"), off)
    with pytest.raises(ube.UbeError, match="unsupported"):
        ube.maxsim(f, f, scores)  # f32 rows
