"""Named model geometries and seeded workloads of the uniform byte encoder.

Geometry fields (zero or missing means "derive the default"):
depth N, hidden D, heads H (head width D/H = 64), ffn F (SwiGLU width), vocab,
context (tokens kept per item), rope_axes (1 text, 2 image, 3 video),
rope_base, rms_epsilon, patch_side, channels, quantization ("bf16"|"e4m3").

The five workloads follow the encoder's documented shapes: byte rows of text at
the trainer's row width, 16x16 RGB patches for images, per-frame 16x16 patches
with a (frame, row, col) grid for video. Sizes are synthetic stand-ins: the
documentation's evaluation sets and checkpoints are not used.
"""
from __future__ import annotations

DEFAULTS = dict(vocab=258, context=1024, rope_axes=1, rope_base=10000.0, rms_epsilon=1e-6,
                patch_side=16, channels=3, quantization="bf16", modality="text", token_width=0)

GEOMETRIES = {
    "tiny": dict(depth=2, hidden=128, heads=2, ffn=512, vocab=256, context=1024, token_width=128),
    "text512": dict(depth=12, hidden=512, heads=8, ffn=1536, vocab=258, context=1024, token_width=128),
    "text512_4k": dict(depth=12, hidden=512, heads=8, ffn=1536, vocab=258, context=4096, token_width=128),
    "image768": dict(depth=12, hidden=768, heads=12, ffn=2304, rope_axes=2, context=1024, modality="image"),
    # shallow text encoders at the widths of the pages' wider tiers (training parity cases)
    "text768_shallow": dict(depth=2, hidden=768, heads=12, ffn=2304, vocab=258, context=1024),
    "text1024_shallow": dict(depth=2, hidden=1024, heads=16, ffn=3072, vocab=258, context=1024),
    "video1024": dict(depth=24, hidden=1024, heads=16, ffn=3072, rope_axes=3, context=2048, modality="video"),
    "video1024_e4m3": dict(depth=24, hidden=1024, heads=16, ffn=3072, rope_axes=3, context=2048,
                           modality="video", quantization="e4m3"),
}

# input recipes (seed 1)
WORKLOADS = {
    "tiny": dict(geometry="tiny", input="text", count=8, len_lo=16, len_hi=65, byte_lo=0, byte_hi=256),
    "ragged": dict(geometry="text512", input="text", count=64, len_lo=1, len_hi=1025, byte_lo=32, byte_hi=127),
    "ragged_trunc": dict(geometry="text512", input="text", count=64, len_lo=1, len_hi=2049, byte_lo=32,
                         byte_hi=127),
    "throughput": dict(geometry="text512", input="text", count=1024, fixed_length=1024, byte_lo=0, byte_hi=256),
    # the pages' text-only row width: 4096-byte rows, attention about half the flops
    "long": dict(geometry="text512_4k", input="text", count=256, fixed_length=4096, byte_lo=0, byte_hi=256),
    # many short segments (the pages pack sentences of a few hundred bytes), about the throughput token budget
    "packed": dict(geometry="text512", input="text", count=4096, len_lo=32, len_hi=513, byte_lo=32, byte_hi=127),
    # one device's training step as the pages' trainer example sizes it: 64 rows of 1024 bytes
    "train": dict(geometry="text512", input="text", count=64, fixed_length=1024, byte_lo=0, byte_hi=256),
    "image": dict(geometry="image768", input="media", count=128, frames=1, height=256, width=256),
    "video": dict(geometry="video1024", input="media", count=16, frames=8, height=224, width=224),
    "video_e4m3": dict(geometry="video1024_e4m3", input="media", count=16, frames=8, height=224, width=224),
}


def complete(geometry: dict) -> dict:
    g = dict(DEFAULTS)
    for k, v in geometry.items():
        if v is None or (k in DEFAULTS and v == 0):
            continue  # zero means "derive the default" for defaulted fields
        g[k] = v
    if "heads" not in g or not g["heads"]:
        g["heads"] = g["hidden"] // 64
    if "ffn" not in g or not g["ffn"]:
        g["ffn"] = 3 * g["hidden"]
    return g


def geometry(name: str) -> dict:
    return complete(GEOMETRIES[name])


def patch_dim(g: dict) -> int:
    return g["patch_side"] * g["patch_side"] * g["channels"]


def block_flops(g: dict, tokens: int, sum_sq_lengths: int) -> float:
    """Dense multiply-add flops (2 per MAC) of the N blocks over a batch."""
    D, F, N = g["hidden"], g["ffn"], g["depth"]
    gemm = 2.0 * tokens * (D * 3 * D + D * D + D * 2 * F + F * D)
    attn = 2.0 * 2.0 * sum_sq_lengths * D  # q.k and p.v over all heads
    return N * (gemm + attn)


def encode_flops(g: dict, lengths) -> float:
    """Algorithmic flops of one encode: frontend GEMM (media) + blocks + reassociated pool."""
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    ssq = sum(x * x for x in lengths)
    D, H = g["hidden"], g["heads"]
    total = block_flops(g, T, ssq)
    if g.get("modality", "text") != "text":
        total += 2.0 * T * patch_dim(g) * D
    # pool: scores x.u_h (H dot products of D per token), weighted sum (H x D per token),
    # then per item the H x (D x 64) value projection.
    total += 2.0 * T * H * D * 2 + 2.0 * len(lengths) * D * D
    return total


# Contrastive (SigLIP-form, Matryoshka) loss over pooled embeddings: one device's anchors scored against
# every item of the step. ``items`` embeddings of width ``columns``; anchors are items
# [anchor_begin, anchor_begin + anchors); the positives pair item 2k with 2k + 1, and every anchor also
# carries ``hard`` named repel edges and ``ignored`` ignore edges. Starting temperature and bias as the
# pages derive them for the sigmoid form (10 and -10).
SIGLIP_WORKLOADS = {
    "siglip_tiny": dict(items=40, columns=128, anchor_begin=0, anchors=40, widths=(64, 128), hard=1, ignored=1),
    "siglip_small": dict(items=300, columns=256, anchor_begin=0, anchors=300, widths=(64, 128, 256), hard=2,
                         ignored=1),
    "siglip_offset": dict(items=520, columns=256, anchor_begin=130, anchors=200, widths=(64, 192), hard=2,
                          ignored=2),
    # the encoder's own pooled width over a packed step of 4096 segments, every item an anchor
    "siglip_pooled": dict(items=4096, columns=512, anchor_begin=0, anchors=4096, widths=(64, 128, 256, 512),
                          hard=2, ignored=1),
    # one device's band of a 72-device domain: 1024 anchors against 72 x 1024 gathered 1024-d embeddings
    "siglip_band": dict(items=73728, columns=1024, anchor_begin=0, anchors=1024, widths=(64, 128, 256, 512, 1024),
                        hard=2, ignored=1),
}
SIGLIP_TEMPERATURE = 10.0
SIGLIP_BIAS = -10.0


def siglip_flops(items: int, anchors: int, columns: int) -> float:
    """Algorithmic MFMA flops of one loss + gradient pass: the anchor-by-item products at full width,
    then the two gradient contractions (rows and columns), each 2 * anchors * items * columns."""
    return 3.0 * 2.0 * anchors * items * columns
