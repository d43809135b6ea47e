"""Pins of the CPU oracle against what the documentation pages and mathematics fix.

Each test checks the oracle against something other than itself: a value the
pages print (fixtures under tests/golden/), a closed form, an invariant, a
special case that reduces to a textbook routine, or brute force on a tiny case.
Every test is chosen so that a plausible slip (a dropped gain, a wrong sign or
index, swapped operands) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from multimodal_embeddings_amd import configs, synth

RNG = np.random.default_rng(1234)


# ------------------------------------------------------------------ tape


def test_worked_tape_from_the_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_tape.json")))
    data = np.frombuffer(g["data"].encode(), np.uint8)
    lengths, cu, (trunc, tokens) = oracle.tape_plan(np.array(g["offsets"], np.uint64), 1024)
    assert lengths.tolist() == g["lengths"]
    assert cu.tolist() == [0] + list(np.cumsum(g["lengths"]))
    assert (trunc, tokens) == (g["truncated"], g["tokens"])
    for i, item in enumerate(g["items"]):
        assert bytes(data[g["offsets"][i]:g["offsets"][i + 1]]).decode() == item
    r = g["reading_context_8"]
    lengths, cu, (trunc, tokens) = oracle.tape_plan(np.array(g["offsets"], np.uint64), 8)
    assert lengths.tolist() == r["lengths"] and (trunc, tokens) == (r["truncated"], r["tokens"])


def test_tape_arrow_slice_and_empty_items():
    # Arrow slices may start at a non-zero offset; empty items keep length 0
    lengths, cu, stats = oracle.tape_plan(np.array([3, 10, 10, 20], np.uint64), 8)
    assert lengths.tolist() == [7, 0, 8] and cu.tolist() == [0, 7, 7, 15] and stats == (1, 15)
    lengths, cu, stats = oracle.tape_plan(np.array([5], np.uint64), 8)
    assert lengths.tolist() == [] and cu.tolist() == [0] and stats == (0, 0)


def test_tape_decreasing_offsets_refused():
    with pytest.raises(oracle.OracleError):
        oracle.tape_plan(np.array([0, 5, 4], np.uint64), 8)


def test_tape_random_brute_force():
    for _ in range(20):
        n = int(RNG.integers(0, 30))
        lens = RNG.integers(0, 40, size=n)
        start = int(RNG.integers(0, 5))
        offsets = np.concatenate([[start], start + np.cumsum(lens)]).astype(np.uint64)
        ctx = int(RNG.integers(1, 35))
        lengths, cu, (trunc, tokens) = oracle.tape_plan(offsets, ctx)
        kept = [min(int(x), ctx) for x in lens]
        assert lengths.tolist() == kept
        assert tokens == sum(kept) == int(cu[-1])
        assert trunc == sum(1 for x in lens if x > ctx)
        assert all(cu[i + 1] - cu[i] == kept[i] for i in range(n))


# ------------------------------------------------------------- frontends


def test_byte_gather_recovers_bytes_and_restarts_positions(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "worked_tape.json")))
    data = np.frombuffer(g["data"].encode(), np.uint8)
    offsets = np.array(g["offsets"], np.uint64)
    # an embedding whose row b is (b, 2b, -b): the gathered rows name their byte
    E = np.stack([np.arange(256), 2 * np.arange(256), -np.arange(256)], 1).astype(np.float32)
    lengths, cu, _ = oracle.tape_plan(offsets, 1024)
    x, pos = oracle.embed_text(data, offsets, lengths, cu, E)
    assert bytes(x[:, 0].astype(np.uint8)) == g["data"].encode()
    assert np.array_equal(x[:, 1], 2 * x[:, 0]) and np.array_equal(x[:, 2], -x[:, 0])
    assert pos[:, 0].tolist() == list(range(14)) + list(range(10))
    assert not pos[:, 1:].any()
    # truncated: first `ctx` bytes of each item
    lengths, cu, _ = oracle.tape_plan(offsets, 8)
    x, pos = oracle.embed_text(data, offsets, lengths, cu, E)
    assert bytes(x[:, 0].astype(np.uint8)) == b"first do" + b"the seco"


def _coordinate_image(frames, H, W):
    """Pixel (f, y, x, ch) = (y + 3x + 7ch + 11f) mod 256: every pixel names its place."""
    f, y, x, c = np.meshgrid(np.arange(frames), np.arange(H), np.arange(W), np.arange(3), indexing="ij")
    return ((y + 3 * x + 7 * c + 11 * f) % 256).astype(np.uint8)


def test_patch_order_and_scale():
    p = 16
    img = _coordinate_image(1, 32, 48)
    K = p * p * 3
    ident = np.eye(K, dtype=np.float32)  # identity projection exposes the patch vector
    x, pos = oracle.embed_patches(img.reshape(-1), 1, 32, 48, 3, p, ident, 2)
    assert x.shape == (2 * 3, K)
    for r in range(2):
        for c in range(3):
            tok = r * 3 + c
            assert pos[tok].tolist() == [r, c, 0]
            for (py, px, ch) in [(0, 0, 0), (5, 9, 2), (15, 15, 1), (7, 0, 1)]:
                k = (py * p + px) * 3 + ch
                assert x[tok, k] == img[0, p * r + py, p * c + px, ch] / 255.0


def test_patch_grid_from_the_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "patch_grid.json")))
    img = np.zeros((g["height"], g["width"], 3), np.uint8)
    W = np.zeros((768, 8), np.float32)
    x, pos = oracle.embed_patches(img.reshape(-1), 1, g["height"], g["width"], 3, 16, W, 2)
    assert x.shape[0] == g["tokens"]
    assert pos[:, 0].max() + 1 == g["grid_rows"] and pos[:, 1].max() + 1 == g["grid_cols"]


def test_video_positions_frame_row_col():
    img = _coordinate_image(2, 32, 32)
    W = np.eye(768, dtype=np.float32)[:, :4]
    x, pos = oracle.embed_patches(img.reshape(-1), 2, 32, 32, 3, 16, W, 3)
    assert pos.tolist() == [[f, r, c] for f in range(2) for r in range(2) for c in range(2)]
    # first patch element of frame 1, patch (1, 0): pixel (1, 16, 0, 0)
    assert x[4 + 2, 0] == img[1, 16, 0, 0] / 255.0


def test_patch_projection_is_linear_in_pixels():
    img = RNG.integers(0, 256, size=(16, 16, 3)).astype(np.uint8)
    W = RNG.standard_normal((768, 5)).astype(np.float32)
    x, _ = oracle.embed_patches(img.reshape(-1), 1, 16, 16, 3, 16, W, 2)
    np.testing.assert_allclose(x[0], (img.reshape(-1) / 255.0) @ W.astype(np.float64), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------- RMSNorm


def test_rmsnorm_unit_gain_mean_square_closed_form():
    eps = 1e-6
    x = RNG.standard_normal((7, 64)) * 1e-3  # mean square ~ eps, so eps matters
    y = oracle.rmsnorm(x, np.ones(64, np.float32), eps)
    ms = (x ** 2).mean(1)
    np.testing.assert_allclose((y ** 2).mean(1), ms / (ms + eps), rtol=1e-12)


def test_rmsnorm_constant_vector_gives_gain():
    eps = 1e-6
    g = (1 + 0.3 * RNG.standard_normal(32)).astype(np.float32)
    for c in (2.5, -0.75, 1e-3):
        y = oracle.rmsnorm(np.full((1, 32), c), g, eps)
        np.testing.assert_allclose(y[0], g.astype(np.float64) * c / math.sqrt(c * c + eps), rtol=1e-13)


def test_rmsnorm_scale_invariant_without_eps():
    x = RNG.standard_normal((3, 48))
    g = (1 + 0.1 * RNG.standard_normal(48)).astype(np.float32)
    np.testing.assert_allclose(oracle.rmsnorm(37.0 * x, g, 0.0), oracle.rmsnorm(x, g, 0.0), rtol=1e-13)


# ------------------------------------------------------------------ RoPE


def test_rope_position_zero_is_identity():
    v = RNG.standard_normal((5, 128))
    out = oracle.rope(v, np.zeros((5, 3), np.int32), 2, 64, 1, 10000.0)
    assert np.array_equal(out, v)


def test_rope_matches_textbook_complex_rotation():
    d, H, T = 64, 3, 9
    v = RNG.standard_normal((T, H * d))
    pos = np.zeros((T, 3), np.int32)
    pos[:, 0] = RNG.integers(0, 3000, size=T)
    out = oracle.rope(v, pos, H, d, 1, 10000.0)
    z = v[:, 0::2] + 1j * v[:, 1::2]  # pairs (2j, 2j+1) as complex numbers
    j = np.arange(d // 2)
    theta = 10000.0 ** (-2.0 * j / d)
    ang = pos[:, :1] * np.tile(theta, H)[None, :]
    zr = z * np.exp(1j * ang)
    np.testing.assert_allclose(out[:, 0::2], zr.real, atol=1e-11)
    np.testing.assert_allclose(out[:, 1::2], zr.imag, atol=1e-11)


def test_rope_hand_value_first_pair():
    v = np.zeros((1, 64))
    v[0, 0] = 1.0
    pos = np.array([[1, 0, 0]], np.int32)
    out = oracle.rope(v, pos, 1, 64, 1, 10000.0)
    assert out[0, 0] == pytest.approx(math.cos(1.0), abs=1e-15)
    assert out[0, 1] == pytest.approx(math.sin(1.0), abs=1e-15)


def test_rope_preserves_pair_norms_and_relative_positions():
    d = 64
    q = RNG.standard_normal((1, d))
    k = RNG.standard_normal((1, d))
    for m, n in [(3, 17), (100, 40), (0, 999)]:
        rq = oracle.rope(q, np.array([[m, 0, 0]], np.int32), 1, d, 1, 10000.0)
        rk = oracle.rope(k, np.array([[n, 0, 0]], np.int32), 1, d, 1, 10000.0)
        rel = oracle.rope(k, np.array([[n - m, 0, 0]], np.int32), 1, d, 1, 10000.0)
        assert float((rq @ rk.T)[0, 0]) == pytest.approx(float((q @ rel.T)[0, 0]), rel=1e-10, abs=1e-10)
        np.testing.assert_allclose(rq[0, 0::2] ** 2 + rq[0, 1::2] ** 2, q[0, 0::2] ** 2 + q[0, 1::2] ** 2,
                                   rtol=1e-12)


def test_mrope_sections():
    assert [oracle.rope_axis_of(j, 64, 1) for j in range(32)] == [0] * 32
    assert [oracle.rope_axis_of(j, 64, 2) for j in range(32)] == [0] * 16 + [1] * 16
    assert [oracle.rope_axis_of(j, 64, 3) for j in range(32)] == [0] * 11 + [1] * 11 + [2] * 10


def test_mrope_two_axes_with_zero_column_rotates_row_section_only():
    d = 64
    v = RNG.standard_normal((4, d))
    pos2 = np.zeros((4, 3), np.int32)
    pos2[:, 0] = [0, 1, 5, 13]
    out2 = oracle.rope(v, pos2, 1, d, 2, 10000.0)
    out1 = oracle.rope(v, pos2, 1, d, 1, 10000.0)
    np.testing.assert_array_equal(out2[:, :32], out1[:, :32])  # pairs 0..15 on the row axis
    np.testing.assert_array_equal(out2[:, 32:], v[:, 32:])  # column axis at 0: untouched
    # the column section uses the same global frequency ladder: pair 16 at col c
    pos_c = np.zeros((1, 3), np.int32)
    pos_c[0, 1] = 7
    out = oracle.rope(v[:1], pos_c, 1, d, 2, 10000.0)
    th = 10000.0 ** (-2.0 * 16 / d)
    z = (v[0, 32] + 1j * v[0, 33]) * np.exp(1j * 7 * th)
    assert out[0, 32] == pytest.approx(z.real, abs=1e-12) and out[0, 33] == pytest.approx(z.imag, abs=1e-12)
    np.testing.assert_array_equal(out[0, :32], v[0, :32])


# ------------------------------------------------------------- attention


def _cu(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint64)


def test_attention_identical_keys_average_values():
    d, H, L = 64, 2, 11
    q = RNG.standard_normal((L, H * d))
    k = np.tile(RNG.standard_normal((1, H * d)), (L, 1))
    v = RNG.standard_normal((L, H * d))
    out = oracle.attention(q, k, v, _cu([L]), H, d)
    np.testing.assert_allclose(out, np.tile(v.mean(0), (L, 1)), rtol=1e-12, atol=1e-13)


def test_attention_single_token_returns_value():
    d, H = 64, 3
    q, k, v = (RNG.standard_normal((1, H * d)) for _ in range(3))
    np.testing.assert_allclose(oracle.attention(q, k, v, _cu([1]), H, d), v, rtol=1e-14)


def test_attention_two_keys_logistic_closed_form():
    d = 64
    q = RNG.standard_normal((2, d))
    k = RNG.standard_normal((2, d))
    v = RNG.standard_normal((2, d))
    out = oracle.attention(q, k, v, _cu([2]), 1, d)
    for t in range(2):
        s0, s1 = q[t] @ k[0] / 8.0, q[t] @ k[1] / 8.0
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        np.testing.assert_allclose(out[t], p0 * v[0] + (1 - p0) * v[1], rtol=1e-12)


def test_attention_shift_of_keys_and_permutation_invariance():
    d, H, L = 64, 2, 9
    q, k, v = (RNG.standard_normal((L, H * d)) for _ in range(3))
    base = oracle.attention(q, k, v, _cu([L]), H, d)
    shifted = oracle.attention(q, k + RNG.standard_normal((1, H * d)), v, _cu([L]), H, d)
    np.testing.assert_allclose(shifted, base, rtol=1e-10, atol=1e-12)
    perm = RNG.permutation(L)
    permuted = oracle.attention(q, k[perm], v[perm], _cu([L]), H, d)
    np.testing.assert_allclose(permuted, base, rtol=1e-12, atol=1e-13)


def test_attention_items_are_isolated():
    d, H = 64, 1
    lens = [5, 7, 3]
    T = sum(lens)
    q, k, v = (RNG.standard_normal((T, H * d)) for _ in range(3))
    base = oracle.attention(q, k, v, _cu(lens), H, d)
    k2, v2 = k.copy(), v.copy()
    k2[5:12] += 3.0
    v2[5:12] *= -2.0
    other = oracle.attention(q, k2, v2, _cu(lens), H, d)
    np.testing.assert_array_equal(other[:5], base[:5])
    np.testing.assert_array_equal(other[12:], base[12:])
    # and each item alone gives the same rows as inside the batch
    alone = oracle.attention(q[5:12], k[5:12], v[5:12], _cu([7]), H, d)
    np.testing.assert_array_equal(alone, base[5:12])


# ---------------------------------------------------------------- SwiGLU


def test_swiglu_zero_gate_is_zero():
    D, F = 8, 12
    h = RNG.standard_normal((4, D))
    Wu = RNG.standard_normal((D, F)).astype(np.float32)
    Wd = RNG.standard_normal((F, D)).astype(np.float32)
    out = oracle.swiglu(h, np.zeros((D, F), np.float32), Wu, Wd)
    assert not out.any()


def test_swiglu_hand_case_gate_vs_up():
    # h = (2, 3): gate picks h0, up picks h1, down is the identity -> (silu(2) * 3, 0)
    h = np.array([[2.0, 3.0]])
    Wg = np.array([[1, 0], [0, 0]], np.float32)
    Wu = np.array([[0, 0], [1, 0]], np.float32)
    Wd = np.eye(2, dtype=np.float32)
    out = oracle.swiglu(h, Wg, Wu, Wd)
    silu2 = 1.7615941559557646  # 2 * logistic(2)
    assert out[0, 0] == pytest.approx(silu2 * 3.0, rel=1e-15)
    assert out[0, 1] == 0.0


# ------------------------------------------------------------------ pool


def _pool_weights(D, rng):
    q = rng.standard_normal(D).astype(np.float32)
    wk = rng.standard_normal((D, D)).astype(np.float32) * 0.1
    wv = rng.standard_normal((D, D)).astype(np.float32) * 0.1
    return q, wk, wv


def test_pool_single_token_is_value_projection():
    D, H = 128, 2
    q, wk, wv = _pool_weights(D, RNG)
    xf = RNG.standard_normal((1, D))
    out = oracle.pool(xf, _cu([1]), H, q, wk, wv)
    np.testing.assert_allclose(out[0], xf[0] @ wv.astype(np.float64), rtol=1e-12)


def test_pool_zero_query_is_mean_of_values():
    D, H, L = 128, 2, 6
    _, wk, wv = _pool_weights(D, RNG)
    xf = RNG.standard_normal((L, D))
    out = oracle.pool(xf, _cu([L]), H, np.zeros(D, np.float32), wk, wv)
    np.testing.assert_allclose(out[0], (xf @ wv.astype(np.float64)).mean(0), rtol=1e-12)


def test_pool_identical_tokens_and_empty_items():
    D, H = 128, 2
    q, wk, wv = _pool_weights(D, RNG)
    row = RNG.standard_normal((1, D))
    xf = np.tile(row, (5, 1))
    out = oracle.pool(xf, _cu([0, 5, 0]), H, q, wk, wv)
    assert not out[0].any() and not out[2].any()
    np.testing.assert_allclose(out[1], row[0] @ wv.astype(np.float64), rtol=1e-12)


def test_pool_two_tokens_closed_form_per_head():
    # W_k = I: head h scores are q_h . xf_t,h / 8; W_v = I: values are xf itself
    D, H = 128, 2
    q = RNG.standard_normal(D).astype(np.float32)
    xf = RNG.standard_normal((2, D))
    I = np.eye(D, dtype=np.float32)
    out = oracle.pool(xf, _cu([2]), H, q, I, I)
    for h in range(H):
        sl = slice(64 * h, 64 * h + 64)
        s = [float(q[sl] @ xf[t, sl]) / 8.0 for t in range(2)]
        p0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        np.testing.assert_allclose(out[0, sl], p0 * xf[0, sl] + (1 - p0) * xf[1, sl], rtol=1e-12)


def test_pool_reassociation_identity():
    # s = xf . (W_k,h q_h) and pooled_h = (sum_t p_t xf_t) W_v,h: exact in real arithmetic
    D, H, L = 128, 2, 13
    q, wk, wv = _pool_weights(D, RNG)
    xf = RNG.standard_normal((L, D))
    out = oracle.pool(xf, _cu([L]), H, q, wk, wv)
    W = wk.astype(np.float64)
    for h in range(H):
        sl = slice(64 * h, 64 * h + 64)
        u = W[:, sl] @ q[sl].astype(np.float64) / 8.0
        s = xf @ u
        p = np.exp(s - s.max())
        p /= p.sum()
        np.testing.assert_allclose(out[0, sl], (p @ xf) @ wv.astype(np.float64)[:, sl], rtol=1e-11)


# ------------------------------------------------------------ whole model


def _tiny_geometry(**kw):
    g = configs.geometry("tiny")
    g.update(kw)
    return g


def test_block_with_zero_out_and_down_projections_is_identity():
    # Net2Net deepening (UForm page, "Pretrained Models & Recipes"): identity blocks
    g = _tiny_geometry(depth=1)
    w = synth.make_weights(g, gain_jitter=0.2)
    synth.set_matrix(w, "w_o", np.zeros((128, 128), np.float32), 0)
    synth.set_matrix(w, "w_down", np.zeros((512, 128), np.float32), 0)
    x0 = RNG.standard_normal((20, 128))
    pos = np.zeros((20, 3), np.int32)
    pos[:, 0] = np.arange(20)
    x, xf = oracle.forward_states(w, x0, pos, _cu([20]))
    assert np.array_equal(x, x0)


def test_depth_zero_single_byte_closed_form():
    # no blocks: pooled(one byte b) = rmsnorm(E[b], g_f) W_v
    g = _tiny_geometry(depth=0)
    w = synth.make_weights(g, gain_jitter=0.3)
    data = np.array([77], np.uint8)
    pooled, stats = oracle.encode_text(w, data, np.array([0, 1], np.uint64))
    e = w.f32["embed"][77].astype(np.float64)
    xf = e * w.f32["final_norm"].astype(np.float64) / math.sqrt((e ** 2).mean() + 1e-6)
    np.testing.assert_allclose(pooled[0], xf @ w.f32["pool_wv"].astype(np.float64), rtol=1e-12, atol=1e-15)
    assert stats == (0, 1)


def test_deepened_model_reproduces_embeddings():
    g = _tiny_geometry(depth=2)
    w = synth.make_weights(g)
    batch = synth.workload_inputs("tiny")
    base, _ = oracle.encode_text(w, batch.data, batch.offsets)
    g3 = _tiny_geometry(depth=3)
    w3 = synth.make_weights(g3)
    for name in ("embed", "pool_query", "pool_wk", "pool_wv"):
        w3.f32[name] = w.f32[name]
    w3.f32["final_norm"] = w.f32["final_norm"]
    order = [0, None, 1]  # identity block inserted in the middle
    for dst, src in enumerate(order):
        for name in ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "attn_norm", "mlp_norm"):
            if src is not None:
                w3.f32[name][dst] = w.f32[name][src]
        if src is None:
            w3.f32["w_o"][dst] = np.zeros_like(w.f32["w_o"][0])
            w3.f32["w_down"][dst] = np.zeros_like(w.f32["w_down"][0])
    grown, _ = oracle.encode_text(w3, batch.data, batch.offsets)
    np.testing.assert_array_equal(grown, base)


def test_encoder_batch_equivariance_and_invariance():
    w = synth.make_weights(configs.geometry("tiny"))
    batch = synth.workload_inputs("tiny")
    base, _ = oracle.encode_text(w, batch.data, batch.offsets)
    perm = [3, 0, 7, 1, 6, 2, 5, 4]
    sub = synth.subset(batch, perm)
    permuted, _ = oracle.encode_text(w, sub.data, sub.offsets)
    np.testing.assert_array_equal(permuted, base[perm])
    alone = synth.subset(batch, [5])
    one, _ = oracle.encode_text(w, alone.data, alone.offsets)
    np.testing.assert_array_equal(one[0], base[5])


def test_encoder_truncation_equals_prefix():
    g = _tiny_geometry(context=40)
    w = synth.make_weights(g)
    rng = np.random.default_rng(5)
    long = rng.integers(0, 256, size=70).astype(np.uint8)
    full, stats = oracle.encode_text(w, long, np.array([0, 70], np.uint64))
    prefix, stats2 = oracle.encode_text(w, long[:40], np.array([0, 40], np.uint64))
    np.testing.assert_array_equal(full, prefix)
    assert stats == (1, 40) and stats2 == (0, 40)


def test_encoder_empty_batch_and_empty_item():
    w = synth.make_weights(configs.geometry("tiny"))
    pooled, stats = oracle.encode_text(w, np.zeros(0, np.uint8), np.array([0], np.uint64))
    assert pooled.shape == (0, 128) and stats == (0, 0)
    data = np.arange(10, dtype=np.uint8)
    pooled, stats = oracle.encode_text(w, data, np.array([0, 4, 4, 10], np.uint64))
    assert not pooled[1].any() and pooled[0].any() and pooled[2].any()


# --------------------------------------------------------------- E4M3


def _all_e4m3_values():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    vals = codes.to(torch.float64).numpy()
    return np.unique(vals[np.isfinite(vals)])


def test_e4m3_codes_round_trip_and_midpoints_match_library_cast():
    vals = _all_e4m3_values()
    assert vals.max() == 448.0 and len(vals) == 253  # 254 finite codes, +0 and -0 merge
    for v in vals:
        assert oracle.e4m3_round(v) == v
    pos = vals[vals >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    probes = np.concatenate([mids, mids * (1 + 2.0 ** -12), mids * (1 - 2.0 ** -12), -mids])  # exact in fp32
    expected = torch.from_numpy(probes).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_round(v) for v in probes])
    np.testing.assert_array_equal(got, expected)


def test_e4m3_saturates_and_qdq_scale():
    assert oracle.e4m3_round(500.0) == 448.0 and oracle.e4m3_round(-1e6) == -448.0
    assert oracle.e4m3_round(2.0 ** -10) == 0.0 and oracle.e4m3_round(3 * 2.0 ** -10) == 2.0 ** -8
    a = RNG.standard_normal(1000)
    r = oracle.e4m3_qdq(a)
    i = int(np.argmax(np.abs(a)))
    assert r[i] == pytest.approx(a[i], rel=1e-15)  # amax maps to the 448 code exactly
    s = np.abs(a).max() / 448.0
    # every output is s times an E4M3 value, and within half a quantum of the input
    q = r / s
    vals = set(_all_e4m3_values().tolist())
    assert all(round(float(abs(x)), 9) in {round(v, 9) for v in vals} for x in q[:50])
    assert np.all(np.abs(r - a) <= np.abs(a) * 2 ** -4 + s * 2 ** -10)
    assert not oracle.e4m3_qdq(np.zeros(8)).any()


def test_bf16_round_matches_library_cast():
    vals = np.concatenate([RNG.standard_normal(2000) * np.exp(RNG.uniform(-20, 20, 2000)),
                           [0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 3.0e38, -1e-39]])
    f32 = vals.astype(np.float32)
    want = torch.from_numpy(f32).to(torch.bfloat16).double().numpy()
    got = np.array([oracle.bf16_round(float(v)) for v in f32])
    np.testing.assert_array_equal(got, want)
    # ties go to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7
    assert oracle.bf16_round(1.0 + 2 ** -8) == 1.0 and oracle.bf16_round(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6


# ------------------------------------------------------- per-token outputs


def _unit_rows(n, width, rng):
    v = rng.standard_normal((n, width))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def test_token_vectors_are_unit_rows_of_the_projection():
    xf = RNG.standard_normal((9, 16))
    w = synth.bf16_bits_to_f32(synth.to_bf16_bits(RNG.standard_normal((16, 8)).astype(np.float32)))
    v = oracle.token_vectors(xf, w)
    assert np.allclose(np.linalg.norm(v, axis=1), 1.0, atol=1e-12)
    # direction: parallel to xf W (cosine 1 against a plain matmul of the same operands)
    y = xf @ w.astype(np.float64)
    assert np.allclose((v * y).sum(1), np.linalg.norm(y, axis=1), rtol=1e-12)
    # identity head: the unit states themselves; positive scaling of W changes nothing; negation flips
    eye = np.eye(16, dtype=np.float32)
    assert np.allclose(oracle.token_vectors(xf, eye), xf / np.linalg.norm(xf, axis=1, keepdims=True), atol=1e-12)
    assert np.allclose(oracle.token_vectors(xf, 4 * w), v, atol=1e-12)
    assert np.allclose(oracle.token_vectors(xf, -w), -v, atol=1e-12)
    # a zero state stays zero (reading) and does not disturb the other rows
    xz = xf.copy()
    xz[3] = 0
    vz = oracle.token_vectors(xz, w)
    assert np.all(vz[3] == 0) and np.allclose(np.delete(vz, 3, 0), np.delete(v, 3, 0))


def test_maxsim_closed_forms():
    e = np.eye(6)
    # one row each: the inner product
    a, b = _unit_rows(1, 6, RNG), _unit_rows(1, 6, RNG)
    assert np.isclose(oracle.maxsim(a, [0, 1], b, [0, 1])[0, 0], float(a[0] @ b[0]), atol=1e-15)
    # orthonormal rows: query {e0, e1} against document {e1, e2} keeps 0 and 1 -> mean 0.5
    assert oracle.maxsim(e[[0, 1]], [0, 2], e[[1, 2]], [0, 2])[0, 0] == 0.5
    # antipodal document: every best match is -1
    q = _unit_rows(5, 6, RNG)
    assert np.isclose(oracle.maxsim(q, [0, 5], -q[:1], [0, 1])[0, 0], -float((q @ q[0]).mean()), atol=1e-15)
    # a document holding every query row scores 1 (the largest inner product of unit rows)
    d = np.concatenate([_unit_rows(7, 6, RNG), q])
    assert np.isclose(oracle.maxsim(q, [0, 5], d, [0, 12])[0, 0], 1.0, atol=1e-12)


def test_maxsim_is_a_mean_of_per_row_maxima():
    # brute force on a tiny case through a different route: sort each query row's
    # products and take the last one
    q, d = _unit_rows(7, 8, RNG), _unit_rows(11, 8, RNG)
    qo, do = [0, 3, 7], [0, 5, 5, 11]
    s = oracle.maxsim(q, qo, d, do)
    for i in range(2):
        for j in range(3):
            rows = d[do[j]:do[j + 1]]
            if len(rows) == 0:
                assert s[i, j] == 0.0  # empty document (reading)
                continue
            best = [sorted(float(np.dot(qt, r)) for r in rows)[-1] for qt in q[qo[i]:qo[i + 1]]]
            assert np.isclose(s[i, j], sum(best) / len(best), atol=1e-14)


def test_maxsim_invariances_and_query_span():
    q, d = _unit_rows(20, 8, RNG), _unit_rows(30, 8, RNG)
    base = oracle.maxsim(q, [0, 20], d, [0, 30], prefix=0, span=64)[0, 0]
    # document rows in any order
    perm = RNG.permutation(30)
    assert np.isclose(oracle.maxsim(q, [0, 20], d[perm], [0, 30])[0, 0], base, atol=1e-14)
    # more document rows never lower a score
    more = np.concatenate([d, _unit_rows(9, 8, RNG)])
    assert oracle.maxsim(q, [0, 20], more, [0, 39])[0, 0] >= base - 1e-14
    # prefix and span select query rows [prefix, prefix + span): the same as slicing them out
    s = oracle.maxsim(q, [0, 20], d, [0, 30], prefix=3, span=5)[0, 0]
    assert np.isclose(s, oracle.maxsim(q[3:8], [0, 5], d, [0, 30], prefix=0, span=64)[0, 0], atol=1e-14)
    # a query with no rows past its prefix scores 0 (reading)
    assert oracle.maxsim(q, [0, 20], d, [0, 30], prefix=20, span=64)[0, 0] == 0.0
    # span caps the counted rows
    s64 = oracle.maxsim(q, [0, 20], d, [0, 30], prefix=0, span=64)[0, 0]
    s20 = oracle.maxsim(q, [0, 20], d, [0, 30], prefix=0, span=20)[0, 0]
    assert s64 == s20
