"""Seeded synthetic weights and inputs for the uniform byte encoder.

This module only draws random numbers and lays them out; it holds none of the
encoder's arithmetic. Both the HIP path and the CPU oracle are fed from it, so
neither re-implements a random generator.

Streams (numpy PCG64 via ``default_rng``):

* weights, seed 0, drawn in this order: the frontend matrix (``embed``
  [vocab x D] for text, ``patch_proj`` [p*p*c x D] for media), then for every
  block ``w_qkv`` [D x 3D], ``w_o`` [D x D], ``w_gate`` [D x F], ``w_up``
  [D x F], ``w_down`` [F x D], then ``pool_query`` [D], ``pool_wk`` [D x D],
  ``pool_wv`` [D x D]. Each is ``standard_normal(float32) * 0.02`` rounded to
  bfloat16 (round-to-nearest-even, by torch's cast). Norm gains are 1.0 (fp32)
  unless a caller asks for random gains (tests do, so that a dropped gain is
  seen).
* inputs, seed 1, per workload (see ``configs.WORKLOADS``).

All matrices use the canonical layout y = x @ W, W row-major [in x out].
"""
from __future__ import annotations

import numpy as np
import torch

from . import configs


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exactly equal float32 values."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


class Weights:
    """One model's weights: ``bits[name]`` (uint16 bf16) and ``f32[name]``.

    Per-block tensors are lists indexed by block. Gains are float32 only.
    """

    def __init__(self, geometry: dict):
        self.geometry = dict(geometry)
        self.bits: dict = {}
        self.f32: dict = {}

    def matrix(self, name, layer=None):
        if layer is None:
            return self.f32[name]
        return self.f32[name][layer]


def _bf16_draw(rng, shape, std):
    raw = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    bits = to_bf16_bits(raw)
    return bits, bf16_bits_to_f32(bits)


def make_weights(geometry: dict, seed: int = 0, std: float = 0.02,
                 gain_jitter: float = 0.0, gain_seed: int = 7) -> Weights:
    """Draw a model's weights in the canonical order.

    ``gain_jitter`` > 0 replaces the unit gains by 1 + jitter * N(0, 1)
    (from a separate stream, so the matrices stay the same).
    """
    g = configs.complete(geometry)
    D, F, N = g["hidden"], g["ffn"], g["depth"]
    rng = np.random.default_rng(seed)
    w = Weights(g)

    def put(name, shape, layer_list=False):
        bits, f32 = _bf16_draw(rng, shape, std)
        if layer_list:
            w.bits.setdefault(name, []).append(bits)
            w.f32.setdefault(name, []).append(f32)
        else:
            w.bits[name] = bits
            w.f32[name] = f32

    if g["modality"] == "text":
        put("embed", (g["vocab"], D))
    else:
        put("patch_proj", (configs.patch_dim(g), D))
    for name in ("w_qkv", "w_o", "w_gate", "w_up", "w_down"):
        w.bits[name] = []
        w.f32[name] = []
    for _ in range(N):
        put("w_qkv", (D, 3 * D), True)
        put("w_o", (D, D), True)
        put("w_gate", (D, F), True)
        put("w_up", (D, F), True)
        put("w_down", (F, D), True)
    put("pool_query", (D,))
    put("pool_wk", (D, D))
    put("pool_wv", (D, D))
    if g.get("token_width"):
        put("token_head", (D, g["token_width"]))

    grng = np.random.default_rng(gain_seed)

    def gain():
        if gain_jitter > 0:
            return (1.0 + gain_jitter * grng.standard_normal(D)).astype(np.float32)
        return np.ones(D, dtype=np.float32)

    w.f32["attn_norm"] = [gain() for _ in range(N)]
    w.f32["mlp_norm"] = [gain() for _ in range(N)]
    w.f32["final_norm"] = gain()
    return w


def set_matrix(w: Weights, name: str, value: np.ndarray, layer=None):
    """Overwrite one matrix with bf16-representable values (tests build special cases)."""
    bits = to_bf16_bits(value)
    f32 = bf16_bits_to_f32(bits)
    if layer is None:
        w.bits[name], w.f32[name] = bits, f32
    else:
        w.bits[name][layer], w.f32[name][layer] = bits, f32


# --------------------------------------------------------------------------- inputs


class TextBatch:
    """A ragged byte tape: ``data`` (uint8) and ``count + 1`` uint64 ``offsets``."""

    def __init__(self, data: np.ndarray, offsets: np.ndarray):
        self.data = np.ascontiguousarray(data, dtype=np.uint8)
        self.offsets = np.ascontiguousarray(offsets, dtype=np.uint64)

    @property
    def count(self):
        return len(self.offsets) - 1


class MediaBatch:
    """Images (frames = 1) or clips: a pixel tape of interleaved u8 RGB plus per-item sizes."""

    def __init__(self, pixels, offsets, heights, widths, frames):
        self.data = np.ascontiguousarray(pixels, dtype=np.uint8)
        self.offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
        self.heights = np.ascontiguousarray(heights, dtype=np.uint64)
        self.widths = np.ascontiguousarray(widths, dtype=np.uint64)
        self.frames = np.ascontiguousarray(frames, dtype=np.uint64)

    @property
    def count(self):
        return len(self.offsets) - 1


def tape_from_items(items) -> TextBatch:
    lengths = [len(x) for x in items]
    offsets = np.zeros(len(items) + 1, dtype=np.uint64)
    offsets[1:] = np.cumsum(lengths, dtype=np.uint64)
    data = np.frombuffer(b"".join(bytes(x) for x in items), dtype=np.uint8) if items else np.zeros(0, np.uint8)
    return TextBatch(data.copy(), offsets)


def text_batch(count, lo, hi, byte_lo, byte_hi, seed=1, fixed_length=None) -> TextBatch:
    """``count`` items; lengths ``integers(lo, hi)`` (or fixed), bytes ``integers(byte_lo, byte_hi)``."""
    rng = np.random.default_rng(seed)
    if fixed_length is not None:
        lengths = np.full(count, fixed_length, dtype=np.int64)
    else:
        lengths = rng.integers(lo, hi, size=count)
    total = int(lengths.sum())
    data = rng.integers(byte_lo, byte_hi, size=total, dtype=np.int64).astype(np.uint8)
    offsets = np.zeros(count + 1, dtype=np.uint64)
    offsets[1:] = np.cumsum(lengths).astype(np.uint64)
    return TextBatch(data, offsets)


def media_batch(count, frames, height, width, channels=3, seed=1) -> MediaBatch:
    """``count`` items of ``frames`` x ``height`` x ``width`` x ``channels`` uniform u8 noise."""
    rng = np.random.default_rng(seed)
    per = frames * height * width * channels
    pixels = rng.integers(0, 256, size=count * per, dtype=np.int64).astype(np.uint8)
    offsets = (np.arange(count + 1, dtype=np.uint64) * np.uint64(per))
    return MediaBatch(pixels, offsets, np.full(count, height), np.full(count, width), np.full(count, frames))


def workload_inputs(name: str, seed: int = 1):
    """The seeded input batch of a named workload (shapes from ``configs.WORKLOADS``)."""
    wl = configs.WORKLOADS[name]
    kind = wl["input"]
    if kind == "text":
        return text_batch(wl["count"], wl.get("len_lo", 0), wl.get("len_hi", 0), wl["byte_lo"], wl["byte_hi"],
                          seed=seed, fixed_length=wl.get("fixed_length"))
    return media_batch(wl["count"], wl["frames"], wl["height"], wl["width"], wl.get("channels", 3), seed=seed)


def subset(batch, rows):
    """Items ``rows`` of a batch, re-packed into a fresh tape (used for sampled parity)."""
    rows = list(rows)
    off = batch.offsets.astype(np.int64)
    parts = [batch.data[off[i]:off[i + 1]] for i in rows]
    lengths = [len(p) for p in parts]
    offsets = np.zeros(len(rows) + 1, dtype=np.uint64)
    offsets[1:] = np.cumsum(lengths).astype(np.uint64) if rows else []
    data = np.concatenate(parts) if parts else np.zeros(0, np.uint8)
    if isinstance(batch, TextBatch):
        return TextBatch(data, offsets)
    return MediaBatch(data, offsets, batch.heights[rows], batch.widths[rows], batch.frames[rows])
