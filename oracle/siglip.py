"""CPU oracle of the Matryoshka sigmoid (SigLIP-form) contrastive loss over pooled embeddings.

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke`` and by the CPU-baseline
leg of ``bench.py``; the product package never imports it, and it shares no code with the HIP path.
Plain numpy in float64, dense [anchors x items] matrices, so it suits steps of a few thousand items.

What it computes (UForm overview page, "Matryoshka-Like Multi-Scale Embedders", the SigLIP equation;
UForm for C training page, ``uform_contrastive_t``, ``uform_negatives_t``, ``uform_pair_loss_form_t``,
``uform_relations_view_t`` and ``uform_edges_view_t``):

* Every Matryoshka width m (ascending, a multiple of 8) scores the cosine of the length-m prefixes:
  s[p, j] = <e_p[:m], e_j[:m]> / (|e_p[:m]| |e_j[:m]|). A prefix of norm zero has cosine 0 with
  everything and passes no gradient.
* Logit z = t * s + b with one (inverse temperature t, bias b) pair.
* Anchors are the items [anchor_begin, anchor_begin + anchors); every item is a candidate. Each
  (anchor, item) cell resolves in the pages' order: an item paired with itself is skipped; an ``ignore``
  edge skips; an ``attract`` edge is a positive of its weight; a ``repel`` edge is a negative of its weight;
  every other cell is a negative of ``ambient_weight`` under ambient negatives and skipped under named ones.
* Cell loss: -w log sigma(z) for a positive, -w log(1 - sigma(z)) for a negative (the sigmoid form).
* Width loss: the cell losses summed over the anchor's row, averaged over anchors. Total loss: the mean
  of the width losses.
* Gradients: with respect to every item's embedding (float, both as anchor and as candidate), to t and to b,
  by the chain rule written out step by step (normalisation backward per prefix).
"""
from __future__ import annotations

import numpy as np

AMBIENT, NAMED = 0, 1


def _softplus(x):
    return np.logaddexp(0.0, x)


def _sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def resolve_cells(items, anchor_begin, anchors, attract, repel, ignore, negatives=AMBIENT, ambient_weight=1.0):
    """Label y (+1 positive, -1 negative, 0 skipped) and weight w of every (anchor, item) cell.

    Edge sets are (offsets[anchors + 1], ids, weights-or-None) in compressed-row form over the anchors.
    Later writes win, so the sets are applied from the lowest precedence to the highest.
    """
    y = np.zeros((anchors, items), dtype=np.int8)
    w = np.zeros((anchors, items), dtype=np.float64)
    if negatives == AMBIENT:
        y[:] = -1
        w[:] = ambient_weight

    def apply(edges, label):
        if edges is None:
            return
        off, ids, wts = edges
        off = np.asarray(off, dtype=np.int64)
        for p in range(anchors):
            for e in range(off[p], off[p + 1]):
                j = int(ids[e])
                y[p, j] = label
                w[p, j] = 1.0 if (wts is None or label == 0) else float(wts[e])

    apply(repel, -1)
    apply(attract, +1)
    apply(ignore, 0)
    for p in range(anchors):
        i = anchor_begin + p
        if i < items:
            y[p, i] = 0
    w[y == 0] = 0.0
    return y, w


def _normalise(x):
    n = np.linalg.norm(x, axis=1, keepdims=True)
    inv = np.divide(1.0, n, out=np.zeros_like(n), where=n > 0)
    return x * inv, inv


def _normalise_backward(xhat, inv, dxhat):
    """d(x / |x|) backward: (dxhat - <xhat, dxhat> xhat) / |x|; zero rows pass nothing."""
    return (dxhat - np.sum(xhat * dxhat, axis=1, keepdims=True) * xhat) * inv


def siglip(emb, anchor_begin, anchors, widths, t, b, attract=None, repel=None, ignore=None,
           negatives=AMBIENT, ambient_weight=1.0):
    """Loss, per-width losses, d loss / d emb [items x columns], d loss / d t, d loss / d b (float64)."""
    e = np.asarray(emb, dtype=np.float64)
    items, columns = e.shape
    widths = [columns] if widths is None else [int(m) for m in widths]
    for a, c in zip(widths, widths[1:]):
        if not a < c:
            raise ValueError("widths must be strictly ascending")
    if any(m % 8 or m <= 0 or m > columns for m in widths):
        raise ValueError("widths must be positive multiples of 8 within the embedding width")
    y, w = resolve_cells(items, anchor_begin, anchors, attract, repel, ignore, negatives, ambient_weight)
    K = len(widths)
    grad = np.zeros_like(e)
    width_losses = np.zeros(K)
    dt = db = 0.0
    if anchors == 0:
        return 0.0, width_losses, grad, 0.0, 0.0
    rows = slice(anchor_begin, anchor_begin + anchors)
    for k, m in enumerate(widths):
        xhat, inv = _normalise(e[:, :m])
        s = xhat[rows] @ xhat.T                       # [anchors x items] cosines of the prefixes
        z = t * s + b
        # -log sigma(y z): positives y = +1, negatives y = -1; skipped cells weigh zero
        cell = w * _softplus(-y * z)
        width_losses[k] = cell.sum() / anchors
        # d/dz of w * softplus(-y z) = w * (sigma(z) - [y = +1]); mean over widths and anchors
        g = w * (_sigmoid(z) - (y == 1)) / (K * anchors)
        db += g.sum()
        dt += (g * s).sum()
        ds = t * g
        d_rows = ds @ xhat                            # d loss / d xhat of each anchor
        d_cols = ds.T @ xhat[rows]                    # d loss / d xhat of each item as a candidate
        dxhat = d_cols
        dxhat[rows] += d_rows
        grad[:, :m] += _normalise_backward(xhat, inv, dxhat)
    return float(width_losses.mean()), width_losses, grad, float(dt), float(db)


def siglip_batch(batch, widths, t, b, negatives=AMBIENT, ambient_weight=1.0):
    """``siglip`` over a seeded ``synth.SiglipBatch``."""
    def edges(x):
        return (x.offsets, x.ids, x.weights)
    return siglip(batch.emb, batch.anchor_begin, batch.anchors, widths, t, b, edges(batch.attract),
                  edges(batch.repel), (batch.ignore.offsets, batch.ignore.ids, None), negatives, ambient_weight)


def siglip_sampled(emb, anchor_begin, anchors, widths, t, b, attract=None, repel=None, ignore=None,
                   negatives=AMBIENT, ambient_weight=1.0, sample=(), block=256):
    """``siglip`` for steps too large for dense [anchors x items] matrices: the loss, width losses, d/dt
    and d/db over every cell, and the gradient rows of the items in ``sample`` only. The same steps in
    the same order, taken over blocks of ``block`` anchors; returns (loss, width_losses, {item: row}, dt, db).
    """
    e = np.asarray(emb, dtype=np.float64)
    items, columns = e.shape
    widths = [columns] if widths is None else [int(m) for m in widths]
    K = len(widths)
    sample = sorted(set(int(i) for i in sample))
    grads = {i: np.zeros(columns) for i in sample}
    width_losses = np.zeros(K)
    dt = db = 0.0
    if anchors == 0:
        return 0.0, width_losses, grads, 0.0, 0.0
    idx = np.asarray(sample, dtype=np.int64)

    def rows_of(edges, lo, hi):
        if edges is None:
            return None
        off, ids, wts = edges
        return (np.asarray(off)[lo:hi + 1], ids, wts)

    for k, m in enumerate(widths):
        xhat, inv = _normalise(e[:, :m])
        d_cols = np.zeros((len(sample), m))
        d_rows = {}
        for lo in range(0, anchors, block):
            hi = min(anchors, lo + block)
            y, w = resolve_cells(items, anchor_begin + lo, hi - lo, rows_of(attract, lo, hi), rows_of(repel, lo, hi),
                                 rows_of(ignore, lo, hi), negatives, ambient_weight)
            rows = slice(anchor_begin + lo, anchor_begin + hi)
            s = xhat[rows] @ xhat.T
            z = t * s + b
            width_losses[k] += (w * _softplus(-y * z)).sum() / anchors
            g = w * (_sigmoid(z) - (y == 1)) / (K * anchors)
            db += g.sum()
            dt += (g * s).sum()
            ds = t * g
            if len(idx):
                d_cols += ds[:, idx].T @ xhat[rows]
            for i in sample:
                if anchor_begin + lo <= i < anchor_begin + hi:
                    d_rows[i] = ds[i - anchor_begin - lo] @ xhat
        for n_, i in enumerate(sample):
            dx = d_cols[n_] + d_rows.get(i, 0.0)
            grads[i][:m] += _normalise_backward(xhat[i:i + 1], inv[i:i + 1], dx[None, :])[0]
    return float(width_losses.mean()), width_losses, grads, float(dt), float(db)
