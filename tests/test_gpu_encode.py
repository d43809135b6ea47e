"""Whole-encoder parity of the HIP path against the CPU oracle, through the C ABI.

Bar (per pooled row): cosine >= 0.999 and max |difference| <= 2e-2 against the
float64 oracle; bookkeeping (stats, rows-view metadata) and batch invariance /
run-to-run determinism are bit-exact.
"""
import numpy as np
import pytest

import oracle
from multimodal_embeddings_amd import configs, synth
from tests import sharp_cases as S
from tests.gpu_util import check_pooled, device_bytes, say

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


def _pooled(rows):
    return rows.tensor().double().cpu().numpy()


# ------------------------------------------------------------------ tiny


def test_tiny_matches_oracle_all_rows(ube):
    import torch
    w, model, arena = _model(ube, "tiny", gain_jitter=0.2)
    batch = synth.workload_inputs("tiny")
    g = w.geometry
    T = int(batch.offsets[-1])
    trace = torch.zeros(((g["depth"] + 1) * T * g["hidden"],), dtype=torch.float32, device="cuda:0")
    rows, stats = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets, trace=trace)
    want, ostats = oracle.encode_text(w, batch.data, batch.offsets)
    assert stats == ostats
    assert (rows.count, rows.columns, rows.stride, rows.scalar) == (8, 128, 512, "f32")
    check_pooled(_pooled(rows), want, "tiny")
    # frontend rows are the embedding rows, exactly
    tr = trace.cpu().numpy().reshape(g["depth"] + 1, T, g["hidden"])
    x0 = w.f32["embed"][batch.data.astype(np.int64)]
    np.testing.assert_array_equal(tr[0], x0)
    # residual stream after every block against the oracle run to that depth
    lengths, cu, _ = oracle.tape_plan(batch.offsets, g["context"])
    x0o, pos = oracle.embed_text(batch.data, batch.offsets, lengths, cu, w.f32["embed"])
    for depth in range(1, g["depth"] + 1):
        wd = synth.Weights(dict(g, depth=depth))
        wd.f32 = {k: (v[:depth] if isinstance(v, list) else v) for k, v in w.f32.items()}
        x_ref, _ = oracle.forward_states(wd, x0o, pos, cu)
        rel = np.linalg.norm(tr[depth] - x_ref) / np.linalg.norm(x_ref)
        say(f"  residual after block {depth}: relative error {rel:.2e}")
        assert rel < 1e-2


def test_tiny_bf16_outputs_and_host_tape(ube):
    w, model, arena = _model(ube, "tiny", gain_jitter=0.2)
    batch = synth.workload_inputs("tiny")
    rows32, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets)
    f32 = _pooled(rows32)
    rows16, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets, outputs_scalar="bf16")
    assert rows16.scalar == "bf16" and rows16.stride == 256
    b16 = _pooled(rows16)
    import torch
    np.testing.assert_array_equal(b16, torch.from_numpy(f32).float().to(torch.bfloat16).double().numpy())
    # a host-resident tape is copied in and gives the same rows
    rows_h, _ = ube.text_encode(model, arena, batch.data, batch.offsets)
    np.testing.assert_array_equal(_pooled(rows_h), f32)


def test_tiny_empty_items_and_empty_batch(ube):
    w, model, arena = _model(ube, "tiny", gain_jitter=0.2)
    data = np.arange(40, dtype=np.uint8)
    offsets = np.array([0, 10, 10, 40, 40], np.uint64)
    rows, stats = ube.text_encode(model, arena, device_bytes(data), offsets)
    got = _pooled(rows)
    want, ostats = oracle.encode_text(w, data, offsets)
    assert stats == ostats == (0, 40)
    assert not got[1].any() and not got[3].any()
    check_pooled(got, want, "tiny-empty-items")
    rows, stats = ube.text_encode(model, arena, device_bytes(np.zeros(1, np.uint8)), np.array([0], np.uint64))
    assert rows.count == 0 and stats == (0, 0)


def test_inputs_inside_the_arena_are_refused(ube):
    w, model, arena = _model(ube, "tiny", gain_jitter=0.2)
    batch = synth.workload_inputs("tiny")
    rows, _ = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets)

    class Inside:
        def data_ptr(self):
            return rows.data

    with pytest.raises(ube.UbeError) as e:
        ube.text_encode(model, arena, Inside(), np.array([0, 16], np.uint64))
    assert e.value.status == "invalid_argument"
    with pytest.raises(ube.UbeError) as e:
        ube.text_encode(model, arena, device_bytes(batch.data), np.array([0, 9, 4], np.uint64))
    assert e.value.status == "invalid_argument"


# ------------------------------------------------------------------ text, depth 12 / hidden 512


def test_ragged_rows_match_oracle(ube):
    w, model, arena = _model(ube, "text512")
    batch = synth.workload_inputs("ragged")
    rows, stats = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets)
    got = _pooled(rows)
    assert stats == oracle.tape_plan(batch.offsets, 1024)[2]
    pick = [0, 5, 17, 33, 63]
    sub = synth.subset(batch, pick)
    want, _ = oracle.encode_text(w, sub.data, sub.offsets)
    say(f"  sampled lengths {np.diff(sub.offsets.astype(np.int64)).tolist()}")
    check_pooled(got[pick], want, "ragged")


def test_ragged_truncation_bookkeeping_and_prefix(ube):
    w, model, arena = _model(ube, "text512")
    batch = synth.workload_inputs("ragged_trunc")
    rows, stats = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets)
    assert stats == oracle.tape_plan(batch.offsets, 1024)[2]
    assert stats[0] > 0
    got = _pooled(rows)
    lens = np.diff(batch.offsets.astype(np.int64))
    i = int(np.argmax(lens))
    # an item past the context pools exactly like its first 1024 bytes
    prefix = batch.data[int(batch.offsets[i]):int(batch.offsets[i]) + 1024]
    rows_p, st = ube.text_encode(model, arena, device_bytes(prefix), np.array([0, 1024], np.uint64))
    assert st == (0, 1024)
    np.testing.assert_array_equal(_pooled(rows_p)[0], got[i])


def test_throughput_batch_sampled_parity_invariance_determinism(ube):
    w, model, arena = _model(ube, "text512")
    batch = synth.workload_inputs("throughput")
    data = device_bytes(batch.data)
    rows, stats = ube.text_encode(model, arena, data, batch.offsets)
    assert stats == (0, 1024 * 1024)
    full = _pooled(rows)
    rows2, _ = ube.text_encode(model, arena, data, batch.offsets)
    np.testing.assert_array_equal(_pooled(rows2), full)  # run to run
    pick = [517, 3, 900]
    sub = synth.subset(batch, pick)
    rows_s, _ = ube.text_encode(model, arena, device_bytes(sub.data), sub.offsets)
    np.testing.assert_array_equal(_pooled(rows_s), full[pick])  # batch invariance
    sample_rows = _sample(1024, 16, seed=3, always=(0, 517, 1023))
    sample = synth.subset(batch, sample_rows)
    want, _ = oracle.encode_text(w, sample.data, sample.offsets)
    check_pooled(full[sample_rows], want, "throughput")


def _sample(n, k, seed, always=()):
    """k seeded distinct item indices out of n, including `always`."""
    rng = np.random.default_rng(seed)
    rest = [int(i) for i in rng.permutation(n) if int(i) not in always]
    return sorted(list(always) + rest[:k - len(always)])


# ------------------------------------------------------------------ media


def test_image_batch_sampled_parity(ube):
    w, model, arena = _model(ube, "image768")
    batch = synth.workload_inputs("image")
    rows, stats = ube.encode(model, arena, _dev(batch))
    assert stats == (0, 128 * 256) and rows.count == 128
    full = _pooled(rows)
    pick = _sample(128, 8, seed=4, always=(0, 77, 127))
    sub = synth.subset(batch, pick)
    want, _ = oracle.encode_media(w, sub)
    check_pooled(full[pick], want, "image")
    rows_s, _ = ube.encode(model, arena, _dev(sub))
    np.testing.assert_array_equal(_pooled(rows_s), full[pick])


def test_image_shape_refusals(ube):
    w, model, arena = _model(ube, "image768")
    px = np.zeros(40 * 48 * 3, np.uint8)
    with pytest.raises(ube.UbeError) as e:
        ube.image_encode_pixels(model, arena, device_bytes(px), [0, px.size], [40], [48])
    assert e.value.status == "shape_mismatch"
    big = np.zeros(528 * 528 * 3, np.uint8)  # 33 x 33 = 1089 patches > 1024
    with pytest.raises(ube.UbeError) as e:
        ube.image_encode_pixels(model, arena, device_bytes(big), [0, big.size], [528], [528])
    assert e.value.status == "shape_mismatch"


def test_image_edge_cases_empty_single_patch_and_mixed_sizes(ube):
    """An empty batch, a one-patch image (its pooled row is that token's value projection: the pool's
    one-token case), and images of different sizes in one batch (ragged 256-token tiles: 1, 6, 80 and
    256 patches) against the oracle, with batch invariance of a sub-batch."""
    w, model, arena = _model(ube, "image768")
    rows, stats = ube.image_encode_pixels(model, arena, device_bytes(np.zeros(1, np.uint8)), [0], [], [])
    assert rows.count == 0 and stats == (0, 0)
    rng = np.random.default_rng(21)
    sizes = [(16, 16), (32, 48), (128, 160), (256, 256)]
    items = [rng.integers(0, 256, size=h * w_ * 3, dtype=np.int64).astype(np.uint8) for h, w_ in sizes]
    offsets = np.zeros(len(items) + 1, np.uint64)
    offsets[1:] = np.cumsum([len(x) for x in items])
    batch = synth.MediaBatch(np.concatenate(items), offsets, [h for h, _ in sizes], [w_ for _, w_ in sizes],
                             [1] * len(sizes))
    rows, stats = ube.encode(model, arena, _dev(batch))
    assert stats == (0, 1 + 6 + 80 + 256)
    got = _pooled(rows)
    want, _ = oracle.encode_media(w, batch)
    check_pooled(got, want, "image mixed sizes")
    # the one-patch image: the oracle's dense pool of one token returns xf W_v, which the GPU's
    # reassociated pool must reproduce
    x0, pos, cu = oracle.media_frontend(w, synth.subset(batch, [0]))
    _, xf = oracle.forward_states(w, x0, pos, cu)
    np.testing.assert_allclose(want[0], xf[0] @ w.f32["pool_wv"].astype(np.float64), rtol=1e-9, atol=1e-12)
    sub = synth.subset(batch, [2, 0])
    rows_s, _ = ube.encode(model, arena, _dev(sub))
    np.testing.assert_array_equal(_pooled(rows_s), got[[2, 0]])


def test_video_small_clips_match_oracle(ube):
    w, model, arena = _model(ube, "video1024")
    batch = synth.media_batch(3, 2, 64, 48, seed=4)  # 2 x 4 x 3 = 24 tokens per clip
    rows, stats = ube.encode(model, arena, _dev(batch))
    assert stats == (0, 72)
    want, _ = oracle.encode_media(w, batch)
    check_pooled(_pooled(rows), want, "video-small")


def _dev(batch):
    batch.data_device = device_bytes(batch.data)
    return batch


def test_video_e4m3_small_clips_match_oracle_e4m3_mode(ube):
    w, model, arena = _model(ube, "video1024_e4m3")
    assert model.describe()["quantization"] == 4
    batch = synth.media_batch(3, 4, 112, 112, seed=4)  # 4 x 7 x 7 = 196 tokens per clip
    rows, stats = ube.encode(model, arena, _dev(batch))
    got = _pooled(rows)
    want, _ = oracle.encode_media(w, batch)  # the oracle's E4M3 mode (weights and GEMM rows quantised)
    check_pooled(got, want, "video-small-e4m3", e4m3=True)
    # for information: the same clips through the bf16 model of the same weights
    wb, mb, ab = _model(ube, "video1024")
    rows_b, _ = ube.encode(mb, ab, _dev(batch))
    from tests.gpu_util import row_cos
    say(f"  e4m3 vs bf16 pooled cosine: min {row_cos(got, _pooled(rows_b)).min():.5f}")


def _video_full(ube, name):
    w, model, arena = _model(ube, name)
    batch = synth.workload_inputs("video")
    rows, stats = ube.encode(model, arena, _dev(batch))
    assert stats == (0, 16 * 1568) and rows.count == 16
    return w, batch, _pooled(rows)


VIDEO_SAMPLE = [0, 11]


def test_video_full_batch_sampled_parity(ube):
    w, batch, full = _video_full(ube, "video1024")
    sub = synth.subset(batch, VIDEO_SAMPLE)
    want, _ = oracle.encode_media(w, sub)
    check_pooled(full[VIDEO_SAMPLE], want, "video")


def test_video_e4m3_full_batch_sampled_parity(ube):
    w, batch, full = _video_full(ube, "video1024_e4m3")
    sub = synth.subset(batch, VIDEO_SAMPLE)
    want, _ = oracle.encode_media(w, sub)
    from tests.gpu_util import row_cos
    for j, i in enumerate(VIDEO_SAMPLE):
        say(f"  e4m3 clip {i}: cos {row_cos(full[[i]], want[[j]])[0]:.6f}, max |diff| "
            f"{np.abs(full[i] - want[j]).max():.3e}, pooled rms {np.sqrt((want[j] ** 2).mean()):.3e}")
    _, _, full_bf16 = _video_full(ube, "video1024")
    say(f"  e4m3 vs bf16 run, all clips: min cos {row_cos(full, full_bf16).min():.5f}")
    check_pooled(full[VIDEO_SAMPLE], want, "video-e4m3", e4m3=True)


# ------------------------------------------------------------------ pool and rotary that matter
#
# With std-0.02 weights the pool and block softmaxes are nearly uniform; these cases (tests/sharp_cases.py)
# sharpen them, and tests/test_oracle_sensitivity.py shows on the CPU that a mean pool or wrongly wired
# rotary coordinates miss these bars by at least ten times.


@pytest.mark.parametrize("kind", ["text", "image", "video"])
def test_sharp_pool_matches_oracle(ube, kind):
    w, batch = S.pool_case(kind)
    model, arena = ube.Model(w, 0), ube.Arena(0)
    rows, _ = ube.encode(model, arena, _dev(batch))
    x0, pos, cu = S.frontend(w, batch)
    want = oracle.forward(w, x0, pos, cu)
    check_pooled(_pooled(rows), want, f"sharp pool {kind}")
    arena.close()
    model.close()


@pytest.mark.parametrize("kind", ["text", "image", "video"])
def test_sharp_rotary_residual_trace_matches_oracle(ube, kind):
    import torch
    w, batch = S.rotary_case(kind)
    g = w.geometry
    model, arena = ube.Model(w, 0), ube.Arena(0)
    x0, pos, cu = S.frontend(w, batch)
    T, D = x0.shape
    trace = torch.zeros(((g["depth"] + 1) * T * D,), dtype=torch.float32, device="cuda:0")
    ube.encode(model, arena, _dev(batch), trace=trace)
    tr = trace.cpu().numpy().astype(np.float64).reshape(g["depth"] + 1, T, D)
    ref = S.residual_trace(w, x0, pos, cu)
    for d in range(1, g["depth"] + 1):
        rel = np.linalg.norm(tr[d] - ref[d - 1]) / np.linalg.norm(ref[d - 1])
        say(f"  {kind}: residual after block {d}: relative error {rel:.2e} (bar {S.TRACE_REL:.1e})")
        assert rel <= S.TRACE_REL
    arena.close()
    model.close()


# ------------------------------------------------------------------ 4096-byte rows, packed segments


def test_long_rows_at_depth_2_all_rows(ube):
    """Context 4096 (the pages' text row width): full, partial and truncated rows."""
    g = dict(configs.geometry("text512_4k"))
    g["depth"] = 2
    w = synth.make_weights(g)
    model, arena = ube.Model(w, 0), ube.Arena(0)
    rng = np.random.default_rng(11)
    lengths = [4096, 2500, 5000, 1]
    data = rng.integers(0, 256, sum(lengths), dtype=np.uint8)
    offsets = np.zeros(len(lengths) + 1, np.uint64)
    offsets[1:] = np.cumsum(lengths)
    rows, stats = ube.text_encode(model, arena, device_bytes(data), offsets)
    want, ostats = oracle.encode_text(w, data, offsets)
    assert stats == ostats == (1, 4096 + 2500 + 4096 + 1)
    check_pooled(_pooled(rows), want, "long depth 2")
    arena.close()
    model.close()


def test_largest_context_one_block(ube):
    """The largest context the library takes (32767 tokens: positions fill the int16 coordinates and the
    rotary table): one full-context item, one truncated past it and one short item, at hidden 128 and
    depth 1, against the oracle (128 key tiles per query tile in the attention)."""
    g = dict(configs.geometry("tiny"), depth=1, context=32767, token_width=0)
    w = synth.make_weights(g, gain_jitter=0.2)
    model, arena = ube.Model(w, 0), ube.Arena(0)
    rng = np.random.default_rng(12)
    lengths = [32767, 33000, 5]
    data = rng.integers(0, 256, sum(lengths), dtype=np.int64).astype(np.uint8)
    offsets = np.zeros(len(lengths) + 1, np.uint64)
    offsets[1:] = np.cumsum(lengths)
    rows, stats = ube.text_encode(model, arena, device_bytes(data), offsets)
    assert stats == (1, 32767 + 32767 + 5)
    sub = synth.subset(synth.TextBatch(data, offsets), [0, 2])
    want, _ = oracle.encode_text(w, sub.data, sub.offsets)
    got = _pooled(rows)
    check_pooled(got[[0, 2]], want, "context 32767")
    # the truncated item pools exactly like its first 32767 bytes, which is item 0's length
    prefix = data[int(offsets[1]):int(offsets[1]) + 32767]
    rows_p, _ = ube.text_encode(model, arena, device_bytes(prefix), np.array([0, 32767], np.uint64))
    np.testing.assert_array_equal(_pooled(rows_p)[0], got[1])
    arena.close()
    model.close()


def test_long_rows_sampled(ube):
    w, model, arena = _model(ube, "text512_4k")
    batch = synth.workload_inputs("long")
    rows, stats = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets)
    assert stats == (0, 256 * 4096)
    got = _pooled(rows)
    sub = synth.subset(batch, [0])
    want, _ = oracle.encode_text(w, sub.data, sub.offsets)
    check_pooled(got[[0]], want, "long")


def test_packed_segments_sampled_and_batch_invariant(ube):
    w, model, arena = _model(ube, "text512")
    batch = synth.workload_inputs("packed")
    rows, stats = ube.text_encode(model, arena, device_bytes(batch.data), batch.offsets)
    got = _pooled(rows)
    pick = [0, 1, 1000, 2047, 4095]
    sub = synth.subset(batch, pick)
    want, _ = oracle.encode_text(w, sub.data, sub.offsets)
    check_pooled(got[pick], want, "packed")
    # the same segments encoded alone give the same rows, bit for bit
    alone, _ = ube.text_encode(model, arena, device_bytes(sub.data), sub.offsets)
    np.testing.assert_array_equal(_pooled(alone), got[pick])
