"""Per-step parity of the HIP kernels (through the C ABI's step entry points).

Each kernel is checked on seeded inputs against the CPU oracle's function for
the same step (RMSNorm, attention) or, for the bare projection, against a float64
library matmul of the same bf16 operands. Sizes span several tiles and a ragged tail.
"""
import numpy as np
import pytest

import oracle
from multimodal_embeddings_amd import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _bf16(rng, shape, std=1.0):
    bits = synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * np.float32(std))
    return bits, synth.bf16_bits_to_f32(bits).astype(np.float64)


def _to_dev_bf16(bits):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def _from_dev_bf16(t):
    return t.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(300, 384, 512), (1, 128, 64), (513, 256, 1536), (1024, 1536, 512)])
def test_gemm_matches_float64_matmul(M, N, K):
    import multimodal_embeddings_amd as ube
    torch = _torch()
    say(f"gemm M={M} N={N} K={K}")
    rng = np.random.default_rng(M * 7 + N + K)
    Mp = (M + 255) // 256 * 256
    wb, wf = _bf16(rng, (N, K), 1.0 / np.sqrt(K))
    xb, xf = _bf16(rng, (Mp, K))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    ube.step_gemm(_to_dev_bf16(wb), _to_dev_bf16(xb), y, M, N, K)
    torch.cuda.synchronize()
    got = _from_dev_bf16(y)
    ref = xf[:M] @ wf.T
    err = np.abs(got - ref)
    say(f"  max |err| {err.max():.3e}, max rel {(err / (np.abs(ref) + 1e-3)).max():.3e}")
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-4)


@pytest.mark.parametrize("T,D", [(37, 128), (300, 512), (7, 768), (65, 1024)])
def test_rmsnorm_matches_oracle(T, D):
    import multimodal_embeddings_amd as ube
    torch = _torch()
    say(f"rmsnorm T={T} D={D}")
    rng = np.random.default_rng(T + D)
    x = (rng.standard_normal((T, D)) * rng.uniform(0.01, 3, size=(T, 1))).astype(np.float32)
    g = (1 + 0.3 * rng.standard_normal(D)).astype(np.float32)
    h = torch.empty((T, D), dtype=torch.bfloat16, device="cuda:0")
    ube.step_rmsnorm(torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda(), h, T, D, 1e-6)
    torch.cuda.synchronize()
    got = _from_dev_bf16(h)
    ref = oracle.rmsnorm(x.astype(np.float64), g, 1e-6)
    err = np.abs(got - ref)
    say(f"  max |err| {err.max():.3e}")
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6)


@pytest.mark.parametrize("lengths,heads", [([1, 37, 64, 65, 128, 205, 3], 2), ([1024, 1000, 24], 1),
                                           ([0, 5, 0, 300], 3)])
def test_attention_matches_oracle(lengths, heads):
    import multimodal_embeddings_amd as ube
    torch = _torch()
    say(f"attention lengths={lengths} heads={heads}")
    rng = np.random.default_rng(sum(lengths) + heads)
    T = int(sum(lengths))
    W = heads * 64
    Tp = (T + 255) // 256 * 256 + 256
    qb, qf = _bf16(rng, (Tp, W))
    kb, kf = _bf16(rng, (Tp, W))
    vb, vf = _bf16(rng, (T, W))
    vt = np.zeros((W, Tp), np.uint16)
    vt[:, :T] = vb.T
    o = torch.zeros((T, W), dtype=torch.bfloat16, device="cuda:0")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    ube.step_attention(_to_dev_bf16(qb), _to_dev_bf16(kb), W, _to_dev_bf16(vt), Tp, o, W, cu, heads)
    torch.cuda.synchronize()
    got = _from_dev_bf16(o)
    ref = oracle.attention(qf[:T], kf[:T], vf, cu.astype(np.uint64), heads, 64)
    err = np.abs(got - ref)
    say(f"  max |err| {err.max():.3e}, mean {err.mean():.3e}")
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


@pytest.mark.parametrize("top", [3.0, 1000.0])
def test_attention_reference_follows_growing_scores(top):
    """Keys whose scale grows geometrically along each item (0.1 at its first token, `top` at its last), so
    later key tiles score far above the first one: up to ~15 log2 units (weights summing past 2^8 against
    the first tile's reference) or hundreds (2^score overflows against it). The kernel must move its
    reference when a tile's weights sum past 2^8 or overflow and still give the softmax ("UForm" page, One
    Omni Model: bidirectional attention inside each item). At these magnitudes the kernel's bf16 rounding
    of the pre-scaled queries (q log2(e) / 8, rounded once when loaded) moves scores by up to 2^-9 of their
    size, so the oracle is given those same rounded queries: the comparison isolates the reference
    handling."""
    import multimodal_embeddings_amd as ube
    torch = _torch()
    lengths, heads = [1024, 333, 64, 65, 1], 2
    say(f"attention with key scales 0.1 .. {top}, lengths={lengths}")
    rng = np.random.default_rng(int(top) + 7)
    T = int(sum(lengths))
    W = heads * 64
    Tp = (T + 255) // 256 * 256 + 256
    qb, _ = _bf16(rng, (Tp, W))
    pos = np.concatenate([np.arange(n) / max(n - 1, 1) for n in lengths])
    scale = np.ones((Tp, 1), np.float32)
    scale[:T, 0] = 0.1 * (top / 0.1) ** pos
    kb = synth.to_bf16_bits(rng.standard_normal((Tp, W)).astype(np.float32) * scale)
    kf = synth.bf16_bits_to_f32(kb).astype(np.float64)
    vb, vf = _bf16(rng, (T, W))
    vt = np.zeros((W, Tp), np.uint16)
    vt[:, :T] = vb.T
    o = torch.zeros((T, W), dtype=torch.bfloat16, device="cuda:0")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    ube.step_attention(_to_dev_bf16(qb), _to_dev_bf16(kb), W, _to_dev_bf16(vt), Tp, o, W, cu, heads)
    torch.cuda.synchronize()
    got = _from_dev_bf16(o)
    c32 = np.float32(0.18033688011112042)  # log2(e) / 8 as the kernel holds it
    qs = synth.bf16_bits_to_f32(synth.to_bf16_bits(synth.bf16_bits_to_f32(qb) * c32)).astype(np.float64)
    q_eff = qs / (np.log2(np.e) / 8.0)  # the queries whose exact softmax the kernel's weights follow
    ref = oracle.attention(q_eff[:T], kf[:T], vf, cu.astype(np.uint64), heads, 64)
    err = np.abs(got - ref)
    say(f"  max |err| {err.max():.3e}, mean {err.mean():.3e}")
    assert np.all(np.isfinite(got))
    assert err.max() <= 2e-2 and err.mean() <= 2e-3


def test_device_bf16_rounding_is_nearest_even():
    # the kernels' fp32 -> bf16 conversion, checked through the RMSNorm step with
    # unit gain on rows whose normalised values are known exactly in fp32
    import multimodal_embeddings_amd as ube
    torch = _torch()
    rng = np.random.default_rng(11)
    D = 128
    x = rng.standard_normal((64, D)).astype(np.float32)
    h = torch.empty((64, D), dtype=torch.bfloat16, device="cuda:0")
    ube.step_rmsnorm(torch.from_numpy(x).cuda(), torch.ones(D, device="cuda:0"), h, 64, D, 0.0)
    torch.cuda.synchronize()
    got = h.float().cpu().numpy()
    ms = (x.astype(np.float64) ** 2).mean(1, keepdims=True)
    exact = x / np.sqrt(ms)
    want = torch.from_numpy(exact.astype(np.float32)).to(torch.bfloat16).float().numpy()
    # fp32 normalisation may differ from the exact value by a few fp32 ulps, which can
    # move a value across a bf16 rounding boundary only when it sits within them
    close = np.abs(got - want) <= np.abs(want) * 2.0 ** -7
    assert close.all()
    assert (got == want).mean() > 0.999


def _e4m3_values(codes_u8):
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(codes_u8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


@pytest.mark.parametrize("T,W", [(37, 3072), (5, 1024), (300, 512)])
def test_quantize_e4m3_codes_bit_exact(T, W):
    """Per-row E4M3 codes: scale amax/448 and value * (448/amax) in fp32, then the
    oracle's nearest-even E4M3 rounding of that fp32 value (the same decision)."""
    import multimodal_embeddings_amd as ube
    torch = _torch()
    say(f"quantize_e4m3 T={T} W={W}")
    rng = np.random.default_rng(T * W)
    x = rng.standard_normal((T, W)) * np.exp(rng.uniform(-6, 3, size=(T, 1)))
    x[0] = 0.0  # an all-zero row
    xb = synth.to_bf16_bits(x.astype(np.float32))
    x32 = synth.bf16_bits_to_f32(xb)
    codes = torch.empty((T, W), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((T,), dtype=torch.float32, device="cuda:0")
    ube.step_quantize_e4m3(_to_dev_bf16(xb), codes, scales, T, W)
    torch.cuda.synchronize()
    got = _e4m3_values(codes.cpu().numpy())
    amax = np.abs(x32).max(1).astype(np.float32)
    want_scale = np.where(amax > 0, amax / np.float32(448.0), np.float32(0)).astype(np.float32)
    np.testing.assert_array_equal(scales.cpu().numpy(), want_scale)
    q = np.where(amax > 0, np.float32(448.0) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
    v = (x32 * q[:, None]).astype(np.float32)
    want = np.vectorize(oracle.e4m3_round)(v.astype(np.float64))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("M,N,K", [(300, 256, 1024), (513, 768, 3072)])
def test_gemm_e4m3_matches_float64_matmul_of_decoded_codes(M, N, K):
    import multimodal_embeddings_amd as ube
    torch = _torch()
    say(f"gemm_e4m3 M={M} N={N} K={K}")
    rng = np.random.default_rng(M + N + K)
    Mp = (M + 255) // 256 * 256
    wc = rng.integers(0, 256, size=(N, K)).astype(np.uint8)
    wc[(wc & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    xc = rng.integers(0, 256, size=(Mp, K)).astype(np.uint8)
    xc[(xc & 0x7F) == 0x7F] = 0x38
    ws = 0.003
    xs = rng.uniform(0.001, 0.01, size=Mp).astype(np.float32)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    ube.step_gemm_e4m3(torch.from_numpy(wc).cuda(), ws, torch.from_numpy(xc).cuda(), torch.from_numpy(xs).cuda(), y,
                       M, N, K)
    torch.cuda.synchronize()
    got = _from_dev_bf16(y)
    wv = _e4m3_values(wc) * np.float64(np.float32(ws))
    xv = _e4m3_values(xc[:M]) * xs[:M, None].astype(np.float64)
    ref = xv @ wv.T
    err = np.abs(got - ref)
    scale = np.abs(xv) @ np.abs(wv).T
    say(f"  max |err| {err.max():.3e}, max err / sum|products| {(err / scale).max():.3e}")
    # bf16 output rounding plus the fp8 MFMA's own summation, which keeps fewer bits
    # than fp32 (measured <= 0.2% of sum|products|; E4M3 inputs carry 3 mantissa bits)
    assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 4e-3 * scale)


def _positions(kind, M, rng):
    """Coordinates [M x 3] of seeded tokens: text positions restart per item; image (row, col) on a 16 x 16
    grid; video (frame, row, col) on 8 frames of 14 x 14."""
    t = np.arange(M)
    if kind == "text":
        starts = np.sort(rng.choice(np.arange(1, M), size=3, replace=False))
        item_start = np.zeros(M, np.int64)
        for s in starts:
            item_start[s:] = s
        return np.stack([t - item_start, 0 * t, 0 * t], 1)
    if kind == "image":
        u = t % 256
        return np.stack([u // 16, u % 16, 0 * t], 1)
    u = t % 1568
    return np.stack([u // 196, (u // 14) % 14, u % 14], 1)


@pytest.mark.parametrize("M,D,axes,kind", [(300, 128, 1, "text"), (1000, 512, 1, "text"), (700, 768, 2, "image"),
                                           (1700, 1024, 3, "video"), (1, 1024, 3, "video")])
def test_qkv_rotary_matches_oracle_rope(M, D, axes, kind):
    """The QKV product with its rotary epilogue against the oracle's rotation of a float64 product, element by
    element, at one, two and three rotary axes; a rotation with the axes exchanged (or none) misses the bar."""
    import multimodal_embeddings_amd as ube
    torch = _torch()
    say(f"qkv+rotary M={M} D={D} axes={axes} ({kind})")
    rng = np.random.default_rng(M + D + axes)
    Mp = (M + 255) // 256 * 256
    K = D
    wb, wf = _bf16(rng, (3 * D, K), 1.0 / np.sqrt(K))
    xb, xf = _bf16(rng, (Mp, K))
    pos = _positions(kind, M, rng)
    pos4 = np.zeros((M, 4), np.int16)
    pos4[:, :3] = pos
    positions = int(pos.max()) + 1
    qk = torch.empty((M, 2 * D), dtype=torch.bfloat16, device="cuda:0")
    vt = torch.full((D, Mp), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    ube.step_qkv_rotary(_to_dev_bf16(wb), _to_dev_bf16(xb), M, D, K, pos4, axes, 10000.0, positions, qk, vt, Mp)
    torch.cuda.synchronize()
    got = _from_dev_bf16(qk)
    got_v = _from_dev_bf16(vt)
    prod = xf[:M] @ wf.T
    heads = D // 64
    p32 = pos.astype(np.int32)
    ref_q = oracle.rope(prod[:, :D], p32, heads, 64, axes, 10000.0)
    ref_k = oracle.rope(prod[:, D:2 * D], p32, heads, 64, axes, 10000.0)
    ref = np.concatenate([ref_q, ref_k], 1)
    rms = np.sqrt((ref ** 2).mean())
    err = np.abs(got - ref)
    # one bf16 step of the value (rounding alone reaches half of it) plus fp32 cancellation in the rotation
    bar = 2.0 ** -7 * np.abs(ref) + 1e-4 * rms
    say(f"  q|k max |err| {err.max():.3e} (rms {rms:.3f}); worst err / bar {(err / bar).max():.3f}")
    assert np.all(err <= bar)
    # v feature-major, zero past M up to the 256-token boundary
    v_err = np.abs(got_v[:, :M] - prod[:, 2 * D:].T)
    assert np.all(v_err <= 2.0 ** -7 * np.abs(prod[:, 2 * D:].T) + 1e-4 * rms)
    assert not got_v[:, M:Mp].any()
    # teeth: the rotation is not the identity, and exchanging two axes (when there are two) is far off the bar
    if M > 1:
        plain = np.concatenate([prod[:, :D], prod[:, D:2 * D]], 1)
        assert (np.abs(got - plain) > bar).mean() > 0.5
        if axes > 1:
            sw = p32[:, [1, 0, 2]]
            alt = np.concatenate([oracle.rope(prod[:, :D], sw, heads, 64, axes, 10000.0),
                                  oracle.rope(prod[:, D:2 * D], sw, heads, 64, axes, 10000.0)], 1)
            assert (np.abs(got - alt) > bar).mean() > 0.3


def test_qkv_rotary_refuses_coordinates_outside_the_table():
    import multimodal_embeddings_amd as ube
    torch = _torch()
    D = K = 128
    w = torch.zeros((3 * D, K), dtype=torch.bfloat16, device="cuda:0")
    x = torch.zeros((256, K), dtype=torch.bfloat16, device="cuda:0")
    qk = torch.empty((4, 2 * D), dtype=torch.bfloat16, device="cuda:0")
    vt = torch.empty((D, 256), dtype=torch.bfloat16, device="cuda:0")
    pos = np.zeros((4, 4), np.int16)
    pos[2, 1] = 50
    with pytest.raises(ube.UbeError) as e:
        ube.step_qkv_rotary(w, x, 4, D, K, pos, 2, 10000.0, 50, qk, vt, 256)
    assert e.value.status == "invalid_argument"
    pos[2, 1] = -1
    with pytest.raises(ube.UbeError):
        ube.step_qkv_rotary(w, x, 4, D, K, pos, 2, 10000.0, 64, qk, vt, 256)
