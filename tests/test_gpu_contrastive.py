"""Matryoshka sigmoid contrastive loss of the HIP path against the float64 oracle, through the C ABI.

Bars (derived in the design notes from the arithmetic): loss and width losses within 1e-4 relative
(fp32 sums of fp32 per-cell terms); d loss / d t and d loss / d b within 2e-3 relative plus 1e-6
absolute (fp32 sums whose terms cancel between positives and negatives); the embedding gradient per
row cosine >= 0.999 and max |difference| <= 2e-2 of the largest reference entry (the block coefficients
travel as bf16). Loss-only runs equal the loss of full runs bit for bit; repeated runs are bit-identical.
"""
import numpy as np
import pytest

from multimodal_embeddings_amd import configs, synth
from oracle import siglip as S
from tests.gpu_util import COS_MIN, bf16_tensor, row_cos, say

pytestmark = pytest.mark.gpu

T, B = configs.SIGLIP_TEMPERATURE, configs.SIGLIP_BIAS


@pytest.fixture(scope="module")
def ube():
    import multimodal_embeddings_amd as m
    return m


@pytest.fixture(scope="module")
def arena(ube):
    return ube.Arena(0)


def _edges(e, weighted=True):
    return (e.offsets, e.ids, e.weights if weighted else None)


def _gpu(ube, arena, batch, widths, *, grad=True, want_loss=True, negatives="ambient", wa=1.0, t=T, b=B):
    import torch
    emb = bf16_tensor(batch.emb_bits)
    K = len(widths) if widths is not None else 1
    scalars = torch.full((3 + K,), 12345.0, device="cuda:0", dtype=torch.float32)
    g = torch.full(emb.shape, 777.0, device="cuda:0", dtype=torch.float32) if grad else None
    ube.contrastive(arena, emb, scalars, anchor_begin=batch.anchor_begin, anchor_count=batch.anchors, widths=widths,
                    inverse_temperature=t, bias=b, negatives=negatives, ambient_weight=wa,
                    attract=_edges(batch.attract), repel=_edges(batch.repel), ignore=_edges(batch.ignore, False),
                    want_loss=want_loss, gradient=g)
    torch.cuda.synchronize()
    return scalars.cpu().numpy().astype(np.float64), (g.cpu().numpy().astype(np.float64) if grad else None)


def _oracle(batch, widths, negatives="ambient", wa=1.0, t=T, b=B):
    return S.siglip_batch(batch, widths, t, b, S.AMBIENT if negatives == "ambient" else S.NAMED, wa)


def _check(label, sc, g, ref, K):
    loss, wl, rg, dt, db = ref
    say(f"[{label}] loss {sc[0]:.8g} vs {loss:.8g}; dt {sc[1]:.6g} vs {dt:.6g}; db {sc[2]:.6g} vs {db:.6g}")
    assert abs(sc[0] - loss) <= 1e-4 * abs(loss) + 1e-9, label
    assert np.allclose(sc[3:3 + K], wl, rtol=1e-4, atol=1e-9), (label, sc[3:3 + K], wl)
    assert abs(sc[1] - dt) <= 2e-3 * abs(dt) + 1e-6, label
    assert abs(sc[2] - db) <= 2e-3 * abs(db) + 1e-6, label
    if g is not None:
        live = np.abs(rg).max(1) > 0
        cos = row_cos(g[live], rg[live])
        err = np.abs(g - rg).max()
        scale = np.abs(rg).max()
        say(f"[{label}] gradient rows {live.sum()}: min cos {cos.min():.6f}, max |diff| {err:.3e} "
            f"({err / scale:.2e} of the largest entry)")
        assert cos.min() >= COS_MIN, (label, cos.min())
        assert err <= 2e-2 * scale, (label, err, scale)
        assert np.all(g[~live] == 0.0) or np.abs(g[~live]).max() <= 2e-2 * scale


@pytest.mark.parametrize("name", ["siglip_tiny", "siglip_small", "siglip_offset"])
def test_loss_and_gradient_match_oracle(ube, arena, name):
    wl = configs.SIGLIP_WORKLOADS[name]
    batch = synth.siglip_workload(name)
    say(f"[{name}] items {batch.items} columns {batch.columns} anchors {batch.anchor_begin}+{batch.anchors} "
        f"widths {wl['widths']}")
    sc, g = _gpu(ube, arena, batch, wl["widths"])
    _check(name, sc, g, _oracle(batch, wl["widths"]), len(wl["widths"]))


def test_named_negatives_and_ambient_weight(ube, arena):
    batch = synth.siglip_workload("siglip_small")
    widths = (64, 256)
    for negatives, wa in (("named", 1.0), ("ambient", 0.0), ("ambient", 2.5)):
        label = f"{negatives} wa={wa}"
        sc, g = _gpu(ube, arena, batch, widths, negatives=negatives, wa=wa)
        _check(label, sc, g, _oracle(batch, widths, negatives, wa), 2)


def test_full_width_default_and_sharp_temperature(ube, arena):
    batch = synth.siglip_workload("siglip_small")
    sc, g = _gpu(ube, arena, batch, None, t=30.0, b=-3.0)
    _check("full width, t 30", sc, g, _oracle(batch, None, t=30.0, b=-3.0), 1)


def test_loss_only_and_repeat_are_bit_exact(ube, arena):
    batch = synth.siglip_workload("siglip_offset")
    widths = configs.SIGLIP_WORKLOADS["siglip_offset"]["widths"]
    sc1, g1 = _gpu(ube, arena, batch, widths)
    sc2, g2 = _gpu(ube, arena, batch, widths)
    assert np.array_equal(sc1, sc2) and np.array_equal(g1, g2)
    sc3, _ = _gpu(ube, arena, batch, widths, grad=False)
    assert np.array_equal(sc3, sc1)
    sc4, g4 = _gpu(ube, arena, batch, widths, want_loss=False)
    assert np.isnan(sc4[0]) and np.all(np.isnan(sc4[3:])) and sc4[1] == sc1[1] and sc4[2] == sc1[2]
    assert np.array_equal(g4, g1)


def test_degenerate_steps(ube, arena):
    import torch
    batch = synth.siglip_batch(12, 128, 0, 12, seed=4)
    # no anchors: zero loss and gradient
    empty = synth.siglip_batch(12, 128, 5, 0, seed=4)
    sc, g = _gpu(ube, arena, empty, (64, 128))
    assert np.all(sc == 0.0) and np.all(g == 0.0)
    # a single item: only the self pair, which is skipped
    one = synth.siglip_batch(1, 128, 0, 1, seed=4)
    sc, g = _gpu(ube, arena, one, (128,))
    assert np.all(sc[:3] == 0.0) and np.all(g == 0.0)
    # a zero row: its cosines are 0 and it gets no gradient
    bits = batch.emb_bits.copy()
    bits[3] = 0
    zero = synth.SiglipBatch(bits, 0, 12, batch.attract, batch.repel, batch.ignore)
    sc, g = _gpu(ube, arena, zero, (64, 128))
    _check("zero row", sc, g, _oracle(zero, (64, 128)), 2)
    assert np.all(g[3] == 0.0)
    # widths past the largest get no gradient
    sc, g = _gpu(ube, arena, batch, (64,))
    _check("prefix only", sc, g, _oracle(batch, (64,)), 1)
    assert np.all(g[:, 64:] == 0.0)
    del torch


def test_refusals(ube, arena):
    import torch
    batch = synth.siglip_workload("siglip_tiny")
    emb = bf16_tensor(batch.emb_bits)
    sc = torch.zeros(16, device="cuda:0")
    for kw, status in ((dict(widths=(32, 128)), "unsupported"), (dict(widths=(128, 64)), "invalid_argument"),
                       (dict(widths=(64, 136)), "invalid_argument"), (dict(pair_loss="ranked"), "unsupported"),
                       (dict(anchor_begin=30, anchor_count=20), "invalid_argument"),
                       (dict(attract=(np.zeros(41, np.uint64) + np.arange(41) * 0, np.zeros(0, np.uint32), None),
                             anchor_count=40, widths=(64,)), None),
                       (dict(attract=(np.array([0] + [1] * 40, np.uint64), np.array([99], np.uint32), None)),
                        "invalid_argument"),
                       (dict(attract=(np.array([0, 2] + [2] * 39, np.uint64), np.array([5, 5], np.uint32), None)),
                        "invalid_argument")):
        if status is None:
            ube.contrastive(arena, emb, sc, **kw)
            continue
        with pytest.raises(ube.UbeError) as e:
            ube.contrastive(arena, emb, sc, **kw)
        assert e.value.status == status, (kw, e.value.status)
    with pytest.raises(ube.UbeError) as e:
        ube.contrastive(arena, emb.float().to(torch.bfloat16)[:, :96].contiguous(), sc)
    assert e.value.status == "unsupported"


def test_band_full_size_sampled(ube, arena):
    """One device's band at full size (1024 anchors x 73,728 items x 1024 columns, five widths): the loss,
    d/dt and d/db over every cell and sampled gradient rows against the blocked oracle; the radial part of
    every gradient row (zero in exact arithmetic: the loss ignores each item's scale) stays small."""
    import time
    name = "siglip_band"
    wl = configs.SIGLIP_WORKLOADS[name]
    batch = synth.siglip_workload(name)
    sc, g = _gpu(ube, arena, batch, wl["widths"])
    off = batch.attract.offsets.astype(np.int64)
    named = set(int(x) for x in batch.attract.ids[off[0]:off[2]]) | set(int(x) for x in batch.repel.ids[:4])
    sample = sorted({0, 1, 511, 1023, 1024, 40000, 73727} | named)
    t0 = time.time()
    loss, wls, rows, dt, db = S.siglip_sampled(batch.emb, batch.anchor_begin, batch.anchors, wl["widths"], T, B,
                                               _edges(batch.attract), _edges(batch.repel),
                                               _edges(batch.ignore, False), sample=sample)
    say(f"[band] oracle {time.time() - t0:.1f} s; loss {sc[0]:.8g} vs {loss:.8g}; dt {sc[1]:.6g} vs {dt:.6g}; "
        f"db {sc[2]:.6g} vs {db:.6g}")
    assert abs(sc[0] - loss) <= 1e-4 * abs(loss)
    assert np.allclose(sc[3:3 + len(wls)], wls, rtol=1e-4)
    assert abs(sc[1] - dt) <= 2e-3 * abs(dt) + 1e-6 and abs(sc[2] - db) <= 2e-3 * abs(db) + 1e-6
    want = np.stack([rows[i] for i in sample])
    got = g[sample]
    cos = row_cos(got, want)
    err = np.abs(got - want).max()
    scale = np.abs(want).max()
    say(f"[band] sampled rows {sample}: min cos {cos.min():.6f}, max |diff| {err:.3e} ({err / scale:.2e} of max)")
    assert cos.min() >= COS_MIN and err <= 2e-2 * scale
    e = batch.emb.astype(np.float64)
    radial = np.abs((g * e).sum(1)) / np.maximum(np.linalg.norm(g, axis=1) * np.linalg.norm(e, axis=1), 1e-30)
    say(f"[band] largest radial cosine over {len(g)} rows: {radial.max():.2e}")
    assert radial.max() <= 2e-2
