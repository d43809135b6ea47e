"""Seeded encoder cases whose pool and rotary steps matter to the output.

With every weight drawn at std 0.02 the softmax of the pool and of the blocks is
nearly uniform, so an encoder that pooled by the mean or rotated nothing would land
within the parity bar. These cases draw the same seeded weights with sharper
scales ("UForm" page, FAQ "Why attention pooling instead of mean pooling?": mean
pooling is the uniform-attention special case of the pool; "One Omni Model": 1-D,
2-D and 3-D rotary coordinates):

* pool cases: the full encoder of a workload with pool_query ~ N(0, 1) and
  pool_wk std 0.6 (pool logits of std ~10);
* rotary cases: a depth-2 encoder with the q and k columns of every w_qkv at std
  0.1 for media (block logits of std ~10) and 0.05 for text, checked through the residual stream after each
  block, where a wrong rotation shows before later blocks blur it.

The ablations (the same computation with the mean pool, with every position 0, with
two axes exchanged, with the axes rotated) are evaluated with the oracle only, on the
CPU, to show that each misses the GPU bar by at least ten times.
"""
from __future__ import annotations

import numpy as np

import oracle
from multimodal_embeddings_amd import configs, synth

POOL_STD = dict(pool_query_std=1.0, pool_wk_std=0.6)
QK_STD = {"text": 0.05, "image": 0.1, "video": 0.1}  # byte rows repeat tokens, so text takes a milder scale
TRACE_REL = 1.3e-2  # residual-stream bar of the rotary cases (relative Frobenius error after each block)


def pool_case(kind):
    """-> (weights, batch, rows): the workload's model with a sharp pool, and the sampled items."""
    if kind == "text":
        w = synth.make_weights(configs.geometry("text512"), **POOL_STD)
        batch = synth.subset(synth.workload_inputs("ragged"), [0, 5, 17])
    elif kind == "image":
        w = synth.make_weights(configs.geometry("image768"), **POOL_STD)
        batch = synth.subset(synth.workload_inputs("image"), [0, 77])
    else:
        w = synth.make_weights(configs.geometry("video1024"), **POOL_STD)
        batch = synth.media_batch(2, 2, 224, 224, seed=4)
    return w, batch


def rotary_case(kind):
    """-> (weights, batch): a depth-2 model with sharp q and k columns."""
    if kind == "text":
        g = dict(configs.geometry("text512"), depth=2)
        batch = synth.subset(synth.workload_inputs("ragged"), [0, 5, 17])
    elif kind == "image":
        g = dict(configs.geometry("image768"), depth=2)
        batch = synth.subset(synth.workload_inputs("image"), [0, 77])
    else:
        g = dict(configs.geometry("video1024"), depth=2)
        batch = synth.media_batch(2, 2, 224, 224, seed=4)
    return synth.make_weights(g, qk_std=QK_STD[kind], gain_jitter=0.2), batch


def frontend(w, batch):
    """Oracle frontend rows, positions [T x 3] and prefix sums of a case."""
    if isinstance(batch, synth.TextBatch):
        lengths, cu, _ = oracle.tape_plan(batch.offsets, w.geometry["context"])
        x0, pos = oracle.embed_text(batch.data, batch.offsets, lengths, cu, w.f32["embed"])
        return x0, pos, cu
    return oracle.media_frontend(w, batch)


def truncated(w, depth):
    """The first `depth` blocks of a model (same matrices)."""
    wd = synth.Weights(dict(w.geometry, depth=depth))
    wd.f32 = {k: (v[:depth] if isinstance(v, list) else v) for k, v in w.f32.items()}
    wd.bits = {k: (v[:depth] if isinstance(v, list) else v) for k, v in w.bits.items()}
    return wd


def residual_trace(w, x0, pos, cu):
    """Oracle residual stream after each block -> list of [T x D]."""
    return [oracle.forward_states(truncated(w, d), x0, pos, cu)[0] for d in range(1, w.geometry["depth"] + 1)]


def position_ablations(kind, pos):
    """Wrong coordinate wirings of a case: every position 0, and for several axes exchanged or rotated ones."""
    out = {"positions zeroed": np.zeros_like(pos)}
    if kind == "image":
        out["row and column exchanged"] = pos[:, [1, 0, 2]]
    if kind == "video":
        out["row and column exchanged"] = pos[:, [0, 2, 1]]
        out["axes rotated (row, col, frame)"] = pos[:, [1, 2, 0]]
        out["frame and row exchanged"] = pos[:, [1, 0, 2]]
    return out


def mean_pool_weights(w):
    """The same model with a zero pool query: its pool is the mean of the value projections."""
    wm = synth.Weights(w.geometry)
    wm.f32 = dict(w.f32)
    wm.bits = dict(w.bits)
    wm.f32["pool_query"] = np.zeros_like(w.f32["pool_query"])
    wm.bits["pool_query"] = np.zeros_like(w.bits["pool_query"])
    return wm
