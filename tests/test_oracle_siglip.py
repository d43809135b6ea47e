"""Pins of the contrastive-loss oracle against closed forms, brute force and invariances (CPU only).

The oracle (oracle/siglip.py) writes the loss densely with numpy; every test here checks it against
something it does not share code with: hand-derived values, the SigLIP equation evaluated cell by cell in
plain Python, central finite differences of the loss, and symmetries the definition implies.
"""
import math

import numpy as np
import pytest

from multimodal_embeddings_amd import synth
from oracle import siglip as S

T, B = 10.0, -10.0


def _edges(lists, weights=None):
    e = synth.Edges.from_lists(lists, weights)
    return (e.offsets, e.ids, e.weights)


def _sp(x):
    return math.log1p(math.exp(-abs(x))) + max(x, 0.0)


def test_orthogonal_pair_closed_form():
    # two orthonormal items, ambient negatives only: each anchor has one negative of cosine 0 (logit b)
    e = np.array([[1.0, 0, 0, 0, 0, 0, 0, 0], [0, 1.0, 0, 0, 0, 0, 0, 0]])
    loss, wl, g, dt, db = S.siglip(e, 0, 2, None, T, B)
    assert loss == pytest.approx(_sp(B), rel=1e-12)
    sig = 1.0 / (1.0 + math.exp(-B))
    # each cosine moves item 0 along item 1 (and back); both cells of the pair add t * sigma(b) / 2
    assert np.allclose(g[0], T * sig * e[1], rtol=1e-12, atol=0)
    assert np.allclose(g[1], T * sig * e[0], rtol=1e-12, atol=0)
    assert dt == pytest.approx(0.0, abs=1e-15)
    assert db == pytest.approx(sig, rel=1e-12)


def test_identical_positive_pair_closed_form():
    e = np.array([[1.0] + [0.0] * 7, [2.0] + [0.0] * 7])
    att = _edges([[1], [0]])
    loss, wl, g, dt, db = S.siglip(e, 0, 2, None, T, B, attract=att)
    # cosine 1, logit t + b = 0: -log sigma(0) = log 2 per anchor
    assert loss == pytest.approx(math.log(2.0), rel=1e-12)
    assert db == pytest.approx(-0.5, rel=1e-12)
    assert dt == pytest.approx(-0.5, rel=1e-12)
    # parallel vectors: the cosine is at its maximum, the gradient vanishes
    assert np.abs(g).max() < 1e-15


def test_siglip_equation_cell_by_cell():
    # the pages' per-anchor SigLIP sum with one positive per anchor, evaluated with plain loops
    rng = np.random.default_rng(3)
    n, d = 10, 16
    e = rng.standard_normal((n, d))
    partner = [i ^ 1 for i in range(n)]
    loss, wl, g, dt, db = S.siglip(e, 0, n, None, 3.0, -1.5, attract=_edges([[p] for p in partner]))
    total = 0.0
    for p in range(n):
        for j in range(n):
            if j == p:
                continue
            cos = float(e[p] @ e[j]) / math.sqrt(float(e[p] @ e[p]) * float(e[j] @ e[j]))
            z = 3.0 * cos - 1.5
            if j == partner[p]:
                total += -math.log(1.0 / (1.0 + math.exp(-z)))
            else:
                total += -math.log(1.0 - 1.0 / (1.0 + math.exp(-z)))
    assert loss == pytest.approx(total / n, rel=1e-12)


def _fd_case():
    rng = np.random.default_rng(11)
    n, d = 7, 24
    e = rng.standard_normal((n, d))
    e[3, :8] = 0.0  # a zero first prefix
    att = _edges([[1, 5], [0], [3, 6], [2]], [[1.5, 0.5], [1.0], [2.0, 0.75], [1.25]])
    rep = _edges([[4], [2, 6], [], [0, 5]], [[2.0], [0.5, 1.5], [], [1.0, 0.25]])
    ign = _edges([[5], [], [6], [1]])  # overlaps an attract edge of anchors 0 and 2
    return e, dict(anchor_begin=2, anchors=4, widths=(8, 16, 24), attract=att, repel=rep, ignore=ign,
                   ambient_weight=0.7)


@pytest.mark.parametrize("negatives", [S.AMBIENT, S.NAMED])
def test_gradients_match_finite_differences(negatives):
    e, kw = _fd_case()
    t, b = 4.0, -2.0

    def L(ee, tt=t, bb=b):
        return S.siglip(ee, kw["anchor_begin"], kw["anchors"], kw["widths"], tt, bb, kw["attract"], kw["repel"],
                        kw["ignore"], negatives, kw["ambient_weight"])[0]

    loss, wl, g, dt, db = S.siglip(e, kw["anchor_begin"], kw["anchors"], kw["widths"], t, b, kw["attract"],
                                   kw["repel"], kw["ignore"], negatives, kw["ambient_weight"])
    h = 1e-6
    fd = np.zeros_like(e)
    for i in range(e.shape[0]):
        for c in range(e.shape[1]):
            if i == 3 and c < 8:
                continue  # the zero prefix is a kink of the width-8 cosine: no derivative there
            ep, em = e.copy(), e.copy()
            ep[i, c] += h
            em[i, c] -= h
            fd[i, c] = (L(ep) - L(em)) / (2 * h)
    mask = np.ones_like(e, dtype=bool)
    mask[3, :8] = False
    assert np.allclose(g[mask], fd[mask], rtol=1e-6, atol=1e-9)
    # a zero prefix passes nothing through its own width (wider widths still reach those entries)
    only8 = S.siglip(e, kw["anchor_begin"], kw["anchors"], (8,), t, b, kw["attract"], kw["repel"], kw["ignore"],
                     negatives, kw["ambient_weight"])[2]
    assert np.all(only8[3, :8] == 0.0) and np.abs(only8[:, :8]).max() > 0
    assert dt == pytest.approx((L(e, t + h) - L(e, t - h)) / (2 * h), rel=1e-6, abs=1e-10)
    assert db == pytest.approx((L(e, t, b + h) - L(e, t, b - h)) / (2 * h), rel=1e-6, abs=1e-10)


def test_scale_invariance_and_radial_gradient():
    batch = synth.siglip_batch(24, 64, 0, 24, seed=5)
    widths = (16, 40, 64)
    loss, wl, g, dt, db = S.siglip_batch(batch, widths, T, B)
    alpha = np.linspace(0.25, 4.0, 24)[:, None]
    scaled = synth.SiglipBatch.__new__(synth.SiglipBatch)
    scaled.__dict__.update(batch.__dict__)
    scaled.emb = batch.emb * alpha
    loss2, wl2, g2, dt2, db2 = S.siglip_batch(scaled, widths, T, B)
    assert loss2 == pytest.approx(loss, rel=1e-12)
    assert np.allclose(g2 * alpha, g, rtol=1e-9, atol=1e-15)
    # every width's loss is invariant to an item's scale, so the gradient has no radial part
    radial = np.sum(g * batch.emb, axis=1)
    assert np.abs(radial).max() < 1e-12 * np.abs(g).max() * np.abs(batch.emb).max() * 64


def test_prefix_block_permutation_invariance():
    batch = synth.siglip_batch(30, 64, 0, 30, seed=6)
    widths = (16, 48, 64)
    rng = np.random.default_rng(0)
    perm = np.concatenate([rng.permutation(16), 16 + rng.permutation(32), 48 + rng.permutation(16)])
    loss, _, g, dt, db = S.siglip_batch(batch, widths, T, B)
    moved = synth.SiglipBatch.__new__(synth.SiglipBatch)
    moved.__dict__.update(batch.__dict__)
    moved.emb = batch.emb[:, perm]
    loss2, _, g2, dt2, db2 = S.siglip_batch(moved, widths, T, B)
    assert loss2 == pytest.approx(loss, rel=1e-12)
    assert np.allclose(g2, g[:, perm], rtol=1e-9, atol=1e-15)
    # a permutation that crosses a width boundary changes the loss
    bad = np.arange(64)
    bad[[0, 20]] = bad[[20, 0]]
    moved.emb = batch.emb[:, bad]
    assert abs(S.siglip_batch(moved, widths, T, B)[0] - loss) > 1e-6


def test_matryoshka_is_the_mean_of_single_widths():
    batch = synth.siglip_batch(26, 64, 0, 26, seed=8)
    parts = [S.siglip_batch(batch, (m,), T, B) for m in (16, 32, 64)]
    loss, wl, g, dt, db = S.siglip_batch(batch, (16, 32, 64), T, B)
    assert loss == pytest.approx(np.mean([p[0] for p in parts]), rel=1e-12)
    assert np.allclose(wl, [p[0] for p in parts], rtol=1e-12)
    assert np.allclose(g, np.mean([p[2] for p in parts], axis=0), rtol=1e-9, atol=1e-16)
    assert dt == pytest.approx(np.mean([p[3] for p in parts]), rel=1e-9)
    assert db == pytest.approx(np.mean([p[4] for p in parts]), rel=1e-9)
    # a width scores only its prefix
    assert np.all(parts[0][2][:, 16:] == 0.0)


def test_item_permutation_equivariance():
    batch = synth.siglip_batch(20, 32, 0, 20, seed=9)
    perm = np.random.default_rng(1).permutation(20)
    inv = np.argsort(perm)
    loss, _, g, dt, db = S.siglip_batch(batch, (8, 32), T, B)

    def remap(edges, weighted=True):
        lists, wts = [], []
        for p_new in range(20):
            p_old = perm[p_new]
            off = edges.offsets.astype(int)
            ids = edges.ids[off[p_old]:off[p_old + 1]]
            w = edges.weights[off[p_old]:off[p_old + 1]] if edges.weights is not None else np.ones(len(ids))
            order = np.argsort(inv[ids])
            lists.append(inv[ids][order])
            wts.append(w[order])
        return _edges(lists, wts if weighted else None)

    e2 = batch.emb[perm]
    loss2, _, g2, dt2, db2 = S.siglip(e2, 0, 20, (8, 32), T, B, remap(batch.attract), remap(batch.repel),
                                      remap(batch.ignore, False))
    assert loss2 == pytest.approx(loss, rel=1e-12)
    assert np.allclose(g2, g[perm], rtol=1e-9, atol=1e-16)


def test_precedence_and_modes():
    rng = np.random.default_rng(4)
    e = rng.standard_normal((5, 16))
    # anchor 0 names item 1 in all three sets, item 2 in attract and repel, item 3 only in repel
    att = _edges([[1, 2]], [[2.0, 3.0]])
    rep = _edges([[1, 2, 3]], [[5.0, 7.0, 0.5]])
    ign = _edges([[1]])
    y, w = S.resolve_cells(5, 0, 1, att, rep, ign)
    assert list(y[0]) == [0, 0, 1, -1, -1] and list(w[0]) == [0.0, 0.0, 3.0, 0.5, 1.0]
    y, w = S.resolve_cells(5, 0, 1, att, rep, ign, negatives=S.NAMED)
    assert list(y[0]) == [0, 0, 1, -1, 0] and list(w[0]) == [0.0, 0.0, 3.0, 0.5, 0.0]
    # zero ambient weight is the named mode; doubling every weight doubles the loss (five anchors now)
    att = _edges([[1, 2]] + [[]] * 4, [[2.0, 3.0]] + [[]] * 4)
    rep = _edges([[1, 2, 3]] + [[4]] * 4, [[5.0, 7.0, 0.5]] + [[1.5]] * 4)
    ign = _edges([[1]] + [[]] * 4)
    a = S.siglip(e, 0, 5, (16,), T, B, att, rep, ign, S.AMBIENT, 0.0)
    n = S.siglip(e, 0, 5, (16,), T, B, att, rep, ign, S.NAMED)
    assert a[0] == pytest.approx(n[0], rel=1e-12) and np.allclose(a[2], n[2], rtol=1e-12, atol=0)
    two = S.siglip(e, 0, 5, (16,), T, B, (att[0], att[1], att[2] * 2), (rep[0], rep[1], rep[2] * 2), ign,
                   S.AMBIENT, 2.0)
    one = S.siglip(e, 0, 5, (16,), T, B, att, rep, ign, S.AMBIENT, 1.0)
    assert two[0] == pytest.approx(2 * one[0], rel=1e-12)
    assert np.allclose(two[2], 2 * one[2], rtol=1e-12, atol=0)
    # a self edge is skipped whatever set names it
    self_att = S.siglip(e, 0, 5, (16,), T, B, _edges([[0]] + [[]] * 4), None, None)
    none = S.siglip(e, 0, 5, (16,), T, B, None, None, None)
    assert self_att[0] == pytest.approx(none[0], rel=1e-15)


def test_degenerate_cases():
    e = np.zeros((3, 8))
    e[1, 0] = 1.0
    e[2, 1] = 2.0
    loss, wl, g, dt, db = S.siglip(e, 0, 3, None, T, B)
    # item 0 has no direction: all its cosines are 0 and it gets no gradient
    assert np.all(g[0] == 0.0)
    assert loss == pytest.approx(2 * _sp(B), rel=1e-12)  # every anchor: two negatives at cosine 0
    one = S.siglip(np.ones((1, 8)), 0, 1, None, T, B)
    assert one[0] == 0.0 and np.all(one[2] == 0.0)
    empty = S.siglip(np.ones((4, 8)), 2, 0, None, T, B)
    assert empty[0] == 0.0 and np.all(empty[2] == 0.0) and empty[3] == 0.0 and empty[4] == 0.0


def test_anchor_ranges_add_up():
    # a device's band is a row range: anchors x loss adds over a split of the rows, gradients likewise
    batch = synth.siglip_batch(40, 32, 0, 40, seed=12)
    full = S.siglip_batch(batch, (16, 32), T, B)

    def part(lo, hi):
        sub = synth.siglip_batch(40, 32, 0, 40, seed=12)
        def rows(ed):
            off = ed.offsets.astype(int)
            lists = [ed.ids[off[p]:off[p + 1]] for p in range(lo, hi)]
            w = None if ed.weights is None else [ed.weights[off[p]:off[p + 1]] for p in range(lo, hi)]
            return synth.Edges.from_lists(lists, w)
        sub.anchor_begin, sub.anchors = lo, hi - lo
        sub.attract, sub.repel, sub.ignore = rows(batch.attract), rows(batch.repel), rows(batch.ignore)
        return S.siglip_batch(sub, (16, 32), T, B)

    a, b = part(0, 13), part(13, 40)
    assert 40 * full[0] == pytest.approx(13 * a[0] + 27 * b[0], rel=1e-12)
    assert np.allclose(40 * full[2], 13 * a[2] + 27 * b[2], rtol=1e-9, atol=1e-15)
    assert 40 * full[4] == pytest.approx(13 * a[4] + 27 * b[4], rel=1e-9)


def test_sampled_form_equals_dense_form():
    # the blocked, sampled form used at full size against the dense form on steps both can run
    batch = synth.siglip_batch(90, 64, 17, 50, seed=13)
    edges = dict(attract=(batch.attract.offsets, batch.attract.ids, batch.attract.weights),
                 repel=(batch.repel.offsets, batch.repel.ids, batch.repel.weights),
                 ignore=(batch.ignore.offsets, batch.ignore.ids, None))
    for negatives, wa in ((S.AMBIENT, 1.0), (S.NAMED, 1.0), (S.AMBIENT, 0.4)):
        dense = S.siglip(batch.emb, 17, 50, (16, 48, 64), T, B, negatives=negatives, ambient_weight=wa, **edges)
        sample = [0, 16, 17, 18, 40, 66, 67, 89]
        samp = S.siglip_sampled(batch.emb, 17, 50, (16, 48, 64), T, B, negatives=negatives, ambient_weight=wa,
                                sample=sample, block=7, **edges)
        assert samp[0] == pytest.approx(dense[0], rel=1e-12)
        assert np.allclose(samp[1], dense[1], rtol=1e-12)
        assert samp[3] == pytest.approx(dense[3], rel=1e-10, abs=1e-15)
        assert samp[4] == pytest.approx(dense[4], rel=1e-10, abs=1e-15)
        for i in sample:
            assert np.allclose(samp[2][i], dense[2][i], rtol=1e-9, atol=1e-16), i
