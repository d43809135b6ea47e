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
    raw = rng.standard_normal(size=shape, dtype=np.float32) * np.asarray(std, np.float32)
    bits = to_bf16_bits(raw)
    return bits, bf16_bits_to_f32(bits)


def make_weights(geometry: dict, seed: int = 0, std: float = 0.02,
                 gain_jitter: float = 0.0, gain_seed: int = 7, qk_std: float | None = None,
                 pool_query_std: float | None = None, pool_wk_std: float | None = None) -> Weights:
    """Draw a model's weights in the canonical order.

    ``gain_jitter`` > 0 replaces the unit gains by 1 + jitter * N(0, 1)
    (from a separate stream, so the matrices stay the same).
    ``qk_std`` (the q and k columns of every ``w_qkv``), ``pool_query_std`` and
    ``pool_wk_std`` replace ``std`` for those tensors: the same standard-normal
    draws scaled differently, so that the softmax of the blocks and of the pool
    is sharp (with std 0.02 both are nearly uniform).
    """
    g = configs.complete(geometry)
    D, F, N = g["hidden"], g["ffn"], g["depth"]
    rng = np.random.default_rng(seed)
    w = Weights(g)

    def put(name, shape, layer_list=False, scale=None):
        bits, f32 = _bf16_draw(rng, shape, std if scale is None else scale)
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
    qkv_scale = None
    if qk_std is not None:
        qkv_scale = np.full((1, 3 * D), std, np.float32)
        qkv_scale[0, :2 * D] = qk_std
    for _ in range(N):
        put("w_qkv", (D, 3 * D), True, qkv_scale)
        put("w_o", (D, D), True)
        put("w_gate", (D, F), True)
        put("w_up", (D, F), True)
        put("w_down", (F, D), True)
    put("pool_query", (D,), scale=pool_query_std)
    put("pool_wk", (D, D), scale=pool_wk_std)
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


# --------------------------------------------------------------------------- contrastive loss inputs


class Edges:
    """One edge set in compressed-row form over the anchors: ``offsets`` (anchors + 1, uint64),
    ``ids`` (uint32 item indices, ascending and unique within each run) and optional float32 ``weights``."""

    def __init__(self, offsets, ids, weights=None):
        self.offsets = np.ascontiguousarray(offsets, dtype=np.uint64)
        self.ids = np.ascontiguousarray(ids, dtype=np.uint32)
        self.weights = None if weights is None else np.ascontiguousarray(weights, dtype=np.float32)

    @staticmethod
    def from_lists(lists, weights=None):
        offsets = np.zeros(len(lists) + 1, dtype=np.uint64)
        offsets[1:] = np.cumsum([len(x) for x in lists]).astype(np.uint64) if lists else []
        ids = np.concatenate([np.asarray(x, dtype=np.uint32) for x in lists]) if lists else np.zeros(0, np.uint32)
        w = None
        if weights is not None:
            w = np.concatenate([np.asarray(x, dtype=np.float32) for x in weights]) if weights else \
                np.zeros(0, np.float32)
        return Edges(offsets, ids, w)

    def runs(self):
        off = self.offsets.astype(np.int64)
        for p in range(len(off) - 1):
            ids = self.ids[off[p]:off[p + 1]]
            w = self.weights[off[p]:off[p + 1]] if self.weights is not None else np.ones(len(ids), np.float32)
            yield p, ids, w


class SiglipBatch:
    """Pooled embeddings (bf16 bits and their exact float32 values) plus the relations of one step."""

    def __init__(self, emb_bits, anchor_begin, anchors, attract, repel, ignore):
        self.emb_bits = np.ascontiguousarray(emb_bits, dtype=np.uint16)
        self.emb = bf16_bits_to_f32(self.emb_bits)
        self.anchor_begin = int(anchor_begin)
        self.anchors = int(anchors)
        self.attract, self.repel, self.ignore = attract, repel, ignore

    @property
    def items(self):
        return self.emb_bits.shape[0]

    @property
    def columns(self):
        return self.emb_bits.shape[1]


def siglip_batch(items, columns, anchor_begin, anchors, hard=2, ignored=1, seed=1, weighted=True):
    """Seeded contrastive step: items 2k and 2k + 1 are views of one latent (cosine about 0.8), row norms
    spread over [0.5, 2]; anchor p attracts its partner (and, one time in four, a second random positive),
    repels ``hard`` random items with weights in [0.5, 2] and ignores ``ignored`` random items (which may
    coincide with named edges, so precedence is exercised)."""
    rng = np.random.default_rng(seed)
    latent = rng.standard_normal(size=((items + 1) // 2, columns), dtype=np.float32)
    view = rng.standard_normal(size=(items, columns), dtype=np.float32)
    emb = latent[np.arange(items) // 2] + np.float32(0.5) * view
    emb /= np.linalg.norm(emb, axis=1, keepdims=True) / np.float32(np.sqrt(columns))
    emb *= rng.uniform(0.5, 2.0, size=(items, 1)).astype(np.float32) / np.float32(np.sqrt(columns))
    bits = to_bf16_bits(emb)
    att, att_w, rep, rep_w, ign = [], [], [], [], []
    for p in range(anchors):
        i = anchor_begin + p
        pos = {i ^ 1} if (i ^ 1) < items else set()
        if rng.random() < 0.25:
            pos.add(int(rng.integers(0, items)))
        neg = set(int(x) for x in rng.integers(0, items, size=hard))
        skip = set(int(x) for x in rng.integers(0, items, size=ignored))
        a, r, s = sorted(pos), sorted(neg), sorted(skip)
        att.append(a)
        rep.append(r)
        ign.append(s)
        att_w.append(rng.uniform(0.5, 2.0, size=len(a)) if weighted else np.ones(len(a)))
        rep_w.append(rng.uniform(0.5, 2.0, size=len(r)) if weighted else np.ones(len(r)))
    return SiglipBatch(bits.reshape(items, columns), anchor_begin, anchors,
                       Edges.from_lists(att, att_w), Edges.from_lists(rep, rep_w), Edges.from_lists(ign))


def siglip_workload(name: str, seed: int = 1) -> SiglipBatch:
    wl = configs.SIGLIP_WORKLOADS[name]
    return siglip_batch(wl["items"], wl["columns"], wl["anchor_begin"], wl["anchors"], wl["hard"], wl["ignored"],
                        seed=seed)
