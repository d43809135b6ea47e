"""Throughput of the uniform byte encoder's forward pass on one MI355X.

One step = one whole encode (frontend, N blocks, final norm, attention pool) of
one synthetic batch whose bytes are already resident in HBM. Default workload:
the depth-12 / hidden-512 text encoder on 1024 rows of exactly 1024 bytes.

Prints one JSON line: encoded bytes/s (whole job), pooled embeddings/s,
end-to-end MFMA utilisation, the roofline of the dominant kernel (its launch
durations measured with HIP events on the encode stream during the timed
steps), and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "encoded bytes/sec + MFMA util, depth-12 h512 encoder, 1024-byte rows"
PEAK_BF16 = 2.5e15      # MI355X dense bf16 MFMA, flop/s
PEAK_FP8 = 5.0e15       # MI355X dense fp8 (OCP E4M3) MFMA, flop/s
PEAK_HBM = 8.0e12       # bytes/s

WORKLOAD_TEXT = {
    "throughput": "text encoder depth 12, hidden 512, 8 heads x 64, ffn 1536, 1-axis rotary; 1024 rows x 1024 bytes",
    "ragged": "text encoder depth 12, hidden 512; 64 rows, lengths 1..1024, printable ASCII",
    "long": "text encoder depth 12, hidden 512, context 4096; 256 rows x 4096 bytes",
    "packed": "text encoder depth 12, hidden 512; 4096 segments, lengths 32..512, printable ASCII",
    "tiny": "tiny encoder depth 2, hidden 128; 8 rows, lengths 16..64",
    "image": "image encoder depth 12, hidden 768, 12 heads, 2-axis rotary; 128 images 256x256x3 (256 patches)",
    "video": "video encoder depth 24, hidden 1024, 16 heads, 3-axis rotary; 16 clips 8x224x224x3 (1568 patches)",
    "video_e4m3": "video encoder as above with E4M3 blocks (per-tensor weight scales, per-row activation scales)",
    "maxsim": "hard MaxSim of a 256 x 256 band: token vectors (width 128, bf16) of the first 256 rows of the "
              "1024-byte text batch, queries the first 64 tokens of each row, documents all 1024",
}
MAXSIM_ITEMS = 256
WORKLOAD_TEXT.update({
    "train": "training step of the depth-12 hidden-512 text encoder on 64 rows x 1024 bytes: encode, Matryoshka "
             "sigmoid contrastive loss over the 64 pooled rows (pairs 2k/2k+1, widths 64..512), backward over "
             "the forward's kept activations (norm outputs and gate/up pre-activations rebuilt per block), "
             "Adafactor update of every tensor",
    "siglip_band": "Matryoshka sigmoid contrastive loss + gradient: 1024 anchors (one device's share) against "
                   "73,728 gathered 1024-d bf16 pooled embeddings, widths 64/128/256/512/1024, t 10, b -10, "
                   "ambient negatives, 1-2 positives, 2 hard negatives and 1 ignore edge per anchor",
    "siglip_pooled": "Matryoshka sigmoid contrastive loss + gradient over a 4096-segment step of 512-d pooled "
                     "embeddings, every item an anchor, widths 64/128/256/512",
})
# Contrastive cells: the per-(anchor, item, width) work the method needs at the least -- logit from the
# prefix dot (2 fp32 ops), sigmoid (exp and reciprocal: 2 transcendental + 2 ops), loss (log: 1
# transcendental + 1 op), gradient coefficient (1 op), the row, column and bias sums (4 ops): 10 VALU
# slots plus 3 transcendental ops at a quarter of the VALU rate (12 slots). MI355X issues 64 fp32 lane
# ops per clock per CU (4 SIMDs x 16 lanes), 256 CUs at 2.4 GHz: 3.93e13 slots/s / 22 slots.
CELL_SLOTS = 22
PEAK_CELLS = 256 * 64 * 2.4e9 / CELL_SLOTS


def kernel_flops_per_launch(kernel, g, T, lengths):
    D, F, H = g["hidden"], g["ffn"], g["heads"]
    if kernel == "gemm_gate_up":
        return 2.0 * T * D * 2 * F
    if kernel == "gemm_qkv":
        return 2.0 * T * D * 3 * D
    if kernel == "gemm_down":
        return 2.0 * T * F * D
    if kernel == "gemm_out":
        return 2.0 * T * D * D
    if kernel == "attention":
        return 4.0 * float(np.sum(np.asarray(lengths, np.float64) ** 2)) * D
    if kernel == "gemm_patch":
        return 2.0 * T * g["patch_side"] * g["patch_side"] * g["channels"] * D
    return None  # not a contraction: see kernel_bytes_per_launch


def kernel_bytes_per_launch(kernel, g, T, count):
    """Algorithmic HBM bytes of one launch of a row kernel (what the step must read and write)."""
    D, H = g["hidden"], g["heads"]
    if kernel == "gather":  # byte in; fp32 row, its bf16 copy, the row's sum-of-squares parts, positions out
        return T * (1 + 4 * D + 2 * D + 4 * 16 + 8)
    if kernel == "final_norm":  # fp32 row in; bf16 normalised row and the H pool scores out
        return T * (4 * D + 2 * D + 4 * H)
    if kernel == "pool":  # normalised rows and scores in; pooled fp32 rows out
        return T * (2 * D + 4 * H) + count * D * 4
    raise ValueError(f"no roofline for kernel {kernel}")



def timed_steps(step, steps, stream):
    """Runs `steps` steps between events on `stream` (one event after each step as well) ->
    (mean ms per step over the whole timed region, [ms of each step])."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return ev[0].elapsed_time(ev[-1]) / steps, [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def step_stats(per):
    """Median and minimum of the per-step times (the mean is `ms_per_step`)."""
    import statistics
    return {"ms_step_median": statistics.median(per), "ms_step_min": min(per)} if per else {}

def source_digest(kernel="gemm"):
    h = hashlib.sha256()
    files = ("contrastive.hip", "contrastive.h") if kernel.startswith("contrastive") else ("kernels.hip", "kernels.h")
    for f in files:
        h.update(open(os.path.join(ROOT, "multimodal_embeddings_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(f"{kernel}@{workload}")
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads(n):
    """Sets the OpenMP thread count of the oracle's runtime (libgomp, shared with the oracle library)."""
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def _oracle_units(workload, weights, sub):
    import oracle
    if workload in ("throughput", "ragged", "tiny", "long", "packed"):
        _, stats = oracle.encode_text(weights, sub.data, sub.offsets)
        return stats[1]
    _, stats = oracle.encode_media(weights, sub)
    return int(sub.data.size)


def cpu_baseline(workload, weights, batch, rows):
    """The float64 oracle on the host: a bounded sample on every core, then one short item on one thread."""
    from multimodal_embeddings_amd import synth
    sub = synth.subset(batch, rows)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    _omp_threads(threads)
    t0 = time.perf_counter()
    units = _oracle_units(workload, weights, sub)
    dt = time.perf_counter() - t0
    out = {"value": units / dt, "unit": "bytes/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"items {list(rows)} of the {workload} batch ({units} bytes, float64 oracle, {dt:.1f} s)"}
    # one thread on a short sample: the first 256 bytes of item 0 (text), the first frame of a clip (video),
    # or item 0 (image)
    one = synth.subset(batch, [rows[0]] if rows else [0])
    what = f"item {rows[0] if rows else 0}"
    if isinstance(one, synth.TextBatch) and int(one.offsets[-1]) > 256:
        one = synth.TextBatch(one.data[:256], np.array([0, 256], np.uint64))
        what = f"the first 256 bytes of item {rows[0] if rows else 0}"
    elif not isinstance(one, synth.TextBatch) and int(one.frames[0]) > 1:
        per = int(one.heights[0]) * int(one.widths[0]) * 3
        one = synth.MediaBatch(one.data[:per], np.array([0, per], np.uint64), one.heights, one.widths,
                               np.array([1], np.uint64))
        what = f"the first frame of item {rows[0] if rows else 0}"
    _omp_threads(1)
    t0 = time.perf_counter()
    u1 = _oracle_units(workload, weights, one)
    d1 = time.perf_counter() - t0
    _omp_threads(threads)
    out["one_thread"] = {"value": u1 / d1, "unit": "bytes/s", "sample": f"{what} ({u1} bytes, {d1:.1f} s)"}
    return out


def bench_maxsim(args):
    """Times the MaxSim scorer on token vectors the encoder produced (outside the timed region)."""
    import torch
    import multimodal_embeddings_amd as ube
    from multimodal_embeddings_amd import configs, synth
    g = configs.geometry("text512")
    weights = synth.make_weights(g)
    batch = synth.subset(synth.workload_inputs("throughput"), list(range(MAXSIM_ITEMS)))
    model, arena = ube.Model(weights, 0), ube.Arena(0)
    _, _, vecs, _ = ube.text_encode(model, arena, torch.from_numpy(batch.data).to("cuda:0"), batch.offsets,
                                    outputs_scalar="bf16", outputs=("token_vectors",))
    v = vecs.tensor()
    off_h = vecs.offsets()
    off = torch.from_numpy(off_h.astype(np.int64)).to("cuda:0")
    tape = ube.rows_tape(v, off)
    n = MAXSIM_ITEMS
    scores = torch.empty((n, n), dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    span = 64
    qrows = np.minimum(np.diff(off_h.astype(np.int64)), span)
    drows = np.diff(off_h.astype(np.int64))
    flops = 2.0 * float(qrows.sum()) * float(drows.sum()) * g["token_width"]
    for _ in range(args.warmup):
        ube.maxsim(tape, tape, scores, span=span, completion=1, stream=stream)
    torch.cuda.synchronize()
    ms, per = timed_steps(lambda: ube.maxsim(tape, tape, scores, span=span, completion=1, stream=stream), args.steps,
                          stream)
    achieved = flops / (ms / 1e3) / 1e12
    out = {
        "metric": "MaxSim query-document pairs/sec (256 x 256 band, 64 query tokens x 1024 document tokens, width 128)",
        "value": n * n / (ms / 1e3), "unit": "pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, **step_stats(per), "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (token vectors of the seeded 1024-byte text batch, random-init weights)",
        "config": {"workload": f"maxsim: {WORKLOAD_TEXT['maxsim']}", "pairs": n * n, "parallelism": "1 GPU"},
        "roofline": {"kernel": "maxsim", "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16 / 1e12,
                     "unit": "TFLOP/s", "frac": achieved / (PEAK_BF16 / 1e12), "traffic": None,
                     "avg_launch_ms": ms, "launches": args.steps},
    }
    if not args.no_cpu_baseline:
        import oracle
        host = v.float().cpu().numpy().astype(np.float64)
        nq = 64
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        oracle.maxsim(host, off_h[:nq + 1], host, off_h, prefix=0, span=span)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": nq * n / dt, "unit": "pairs/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"queries 0-{nq - 1} against all {n} documents (float64 oracle, {dt:.1f} s)"}
    else:
        out["cpu_baseline"] = None
    arena.close()
    model.close()
    print(json.dumps(out), flush=True)


def bench_siglip(args):
    """Times whole contrastive calls (loss and gradient) on resident bf16 embeddings."""
    import torch
    import multimodal_embeddings_amd as ube
    from multimodal_embeddings_amd import configs, synth
    wl = configs.SIGLIP_WORKLOADS[args.workload]
    batch = synth.siglip_workload(args.workload)
    emb = torch.from_numpy(batch.emb_bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    widths = wl["widths"]
    K, R, n, D = len(widths), batch.anchors, batch.items, batch.columns
    scalars = torch.zeros(3 + K, dtype=torch.float32, device="cuda:0")
    grad = torch.empty((n, D), dtype=torch.float32, device="cuda:0")
    arena = ube.Arena(0)
    stream = torch.cuda.current_stream()
    rel = dict(attract=(batch.attract.offsets, batch.attract.ids, batch.attract.weights),
               repel=(batch.repel.offsets, batch.repel.ids, batch.repel.weights),
               ignore=(batch.ignore.offsets, batch.ignore.ids, None))

    def step():
        ube.contrastive(arena, emb, scalars, anchor_begin=batch.anchor_begin, anchor_count=R, widths=widths,
                        inverse_temperature=configs.SIGLIP_TEMPERATURE, bias=configs.SIGLIP_BIAS, gradient=grad,
                        completion=1, stream=stream, **rel)

    kernel = args.kernel if args.kernel.startswith("contrastive") else "contrastive_cells"
    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    ube.kernel_timer_start(kernel, args.steps + 4)
    ms, per = timed_steps(step, args.steps, stream)
    kms, launches = ube.kernel_timer_stop()
    per_kernel = {}
    if args.per_kernel:
        for kname in ("contrastive_cells", "contrastive_rows", "contrastive_cols"):
            ube.kernel_timer_start(kname, 8)
            step()
            torch.cuda.synchronize()
            t, nl = ube.kernel_timer_stop()
            per_kernel[kname] = {"ms_per_step": t, "launches": nl}
    avg_s = kms / max(launches, 1) / 1e3
    pairs = R * n
    flops = configs.siglip_flops(n, R, D)
    if kernel == "contrastive_cells":
        achieved = pairs * K / avg_s
        roof = {"kernel": kernel, "bound": "alu", "achieved": achieved / 1e9, "peak": PEAK_CELLS / 1e9,
                "unit": "G cell-widths/s", "frac": achieved / PEAK_CELLS}
    else:
        achieved = 2.0 * R * n * D / avg_s / 1e12
        roof = {"kernel": kernel, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16 / 1e12,
                "unit": "TFLOP/s", "frac": achieved / (PEAK_BF16 / 1e12)}
    roof.update({"traffic": load_traffic(kernel, args.workload), "avg_launch_ms": avg_s * 1e3, "launches": launches})
    out = {
        "metric": "contrastive band pairs/sec (Matryoshka sigmoid loss + gradient over pooled embeddings)",
        "value": pairs / (ms / 1e3), "unit": "pairs/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, **step_stats(per), "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded paired views of shared latents, bf16 rows, seeded edges)",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}", "anchors": R, "items": n,
                   "columns": D, "widths": list(widths), "parallelism": "1 GPU"},
        "mfma_util": flops / (ms / 1e3) / PEAK_BF16,
        "flops_per_step": flops,
        "roofline": roof,
    }
    if per_kernel:
        out["per_kernel_ms"] = per_kernel
    if not args.no_cpu_baseline:
        from oracle import siglip as S
        A = int(args.cpu_rows) if args.cpu_rows else {"siglip_band": 256}.get(args.workload, 1024)
        A = min(A, R)

        def head(e, weighted=True):
            off = e.offsets[:A + 1]
            return (off, e.ids, e.weights if weighted else None)

        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        S.siglip(batch.emb, batch.anchor_begin, A, widths, configs.SIGLIP_TEMPERATURE, configs.SIGLIP_BIAS,
                 head(batch.attract), head(batch.repel), head(batch.ignore, False))
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": A * n / dt, "unit": "pairs/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"anchors 0-{A - 1} against all {n} items, loss and gradient "
                                         f"(float64 oracle, {dt:.1f} s)"}
    else:
        out["cpu_baseline"] = None
    arena.close()
    print(json.dumps(out), flush=True)


def train_flops(g, T, lengths):
    """Model flops of one training step (MFMA work, 2 per multiply-add): the forward once and the backward
    (twice the forward's projections: activation and weight gradients; attention backward counted as 2.5
    times its forward). The rebuilt gate/up projection is recomputation and not counted."""
    from multimodal_embeddings_amd import configs
    fwd = configs.encode_flops(g, lengths)
    attn = 4.0 * float(np.sum(np.asarray(lengths, np.float64) ** 2)) * g["hidden"] * g["depth"]
    bwd = 2.0 * (fwd - attn) + 2.5 * attn
    return fwd + bwd


def bench_train(args):
    """Times whole training steps (encode, contrastive loss, backward, Adafactor) on resident bytes."""
    import torch
    import multimodal_embeddings_amd as ube
    from multimodal_embeddings_amd import configs, synth
    wl = configs.WORKLOADS["train"]
    g = configs.geometry(wl["geometry"])
    weights = synth.make_weights(g)
    batch = synth.workload_inputs("train")
    model, arena, arena2 = ube.Model(weights, 0), ube.Arena(0), ube.Arena(0)
    trainer = ube.Trainer(model, weights, activation_recomputation=args.recompute)
    data = torch.from_numpy(batch.data).to("cuda:0")
    stream = torch.cuda.current_stream()
    n = batch.count
    pairs = synth.Edges.from_lists([[i ^ 1] for i in range(n)])
    widths = (64, 128, 256, 512)
    scalars = torch.zeros(3 + len(widths), device="cuda:0")
    gemb = torch.zeros((n, g["hidden"]), device="cuda:0")

    def step():
        rows, _ = trainer.forward(arena, data, batch.offsets, completion=1, stream=stream)
        emb = torch.as_tensor(rows, device="cuda:0").to(torch.bfloat16)
        ube.contrastive(arena2, emb, scalars, widths=widths, attract=(pairs.offsets, pairs.ids, None),
                        gradient=gemb, completion=1, stream=stream)
        trainer.backward(None, None, None, gemb, completion=1, stream=stream, after_forward=True)
        trainer.step(1e-4, completion=1, stream=stream)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    kernel = args.kernel
    ube.kernel_timer_start(kernel, args.steps * g["depth"] * 8 + 8)
    ms, per = timed_steps(step, args.steps, stream)
    kms, launches = ube.kernel_timer_stop()
    per_kernel = {}
    if args.per_kernel:
        for kname in ube.KERNELS:
            ube.kernel_timer_start(kname, 16 * g["depth"] + 8)
            step()
            torch.cuda.synchronize()
            t, nl = ube.kernel_timer_stop()
            if nl:
                per_kernel[kname] = {"ms_per_step": t, "launches": nl}
    lengths = np.diff(batch.offsets.astype(np.int64))
    T = int(lengths.sum())
    flops = train_flops(g, T, lengths)
    D = g["hidden"]
    if kernel == "attention_bwd":
        kflops = 2.5 * 4.0 * float(np.sum(lengths.astype(np.float64) ** 2)) * D  # one layer's launch pair
    elif kernel == "weight_grad":
        kflops = None
    else:
        kflops = kernel_flops_per_launch(kernel, g, T, lengths) if kernel in ("gemm_qkv", "gemm_out", "gemm_gate_up",
                                                                               "gemm_down", "attention") else None
    avg_s = kms / max(launches, 1) / 1e3
    roof = None
    if kflops:
        achieved = kflops / avg_s / 1e12
        roof = {"kernel": kernel, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s",
                "frac": achieved / (PEAK_BF16 / 1e12), "traffic": load_traffic(kernel, "train"),
                "avg_launch_ms": avg_s * 1e3, "launches": launches}
    out = {
        "metric": "training tokens/sec (one device's step: encode, contrastive loss, backward, Adafactor)",
        "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, **step_stats(per), "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded bytes, random-init bf16 weights N(0, 0.02))",
        "config": {"workload": f"train: {WORKLOAD_TEXT['train']}", "items": n, "tokens": T, "parallelism": "1 GPU",
                   "activation_recomputation": bool(args.recompute)},
        "mfma_util": flops / (ms / 1e3) / PEAK_BF16, "flops_per_step": flops, "roofline": roof,
    }
    if per_kernel:
        out["per_kernel_ms"] = per_kernel
    if not args.no_cpu_baseline:
        from oracle import train as TR
        rows_s = 2
        sub = synth.subset(batch, list(range(rows_s)))
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
        t0 = time.perf_counter()
        TR.text_backward(weights, sub.data, sub.offsets, np.ones((rows_s, D)))
        dt = time.perf_counter() - t0
        toks = int(sub.offsets[-1])
        out["cpu_baseline"] = {"value": toks / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": f"rows 0-{rows_s - 1} ({toks} bytes): float64 forward and autograd backward "
                                         f"({dt:.1f} s; the Adafactor update not included)"}
    else:
        out["cpu_baseline"] = None
    trainer.close()
    arena.close()
    arena2.close()
    model.close()
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="throughput", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--kernel", default=None, help="kernel of the roofline entry (default: the workload's dominant one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", default=None, help="items the CPU oracle encodes (default: ~10-30 s of work)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB device-to-device 3 times (a plain copy kernel of known size, "
                         "for calibrating HBM byte counters)")
    ap.add_argument("--per-kernel", action="store_true", help="also time every kernel kind (extra passes)")
    ap.add_argument("--recompute", action="store_true",
                    help="train: keep only each block's fp32 input and replay the block in the backward")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(items are independent; a multi-GPU run would shard the tape by items)", file=sys.stderr)
        sys.exit(2)

    if args.kernel is None:
        args.kernel = {"train": "attention_bwd"}.get(args.workload, "contrastive_cells" if args.workload.startswith(
            "siglip") else "gemm_gate_up")
    if args.workload == "maxsim":
        return bench_maxsim(args)
    if args.workload.startswith("siglip"):
        return bench_siglip(args)
    if args.workload == "train":
        return bench_train(args)

    import torch
    import multimodal_embeddings_amd as ube
    from multimodal_embeddings_amd import configs, synth

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy probe: 3 copies of {n} bytes (read {n}, write {n} each)", file=sys.stderr, flush=True)
        del src, dst

    wl = configs.WORKLOADS[args.workload]
    g = configs.geometry(wl["geometry"])
    weights = synth.make_weights(g)
    batch = synth.workload_inputs(args.workload)
    model = ube.Model(weights, 0)
    arena = ube.Arena(0)
    batch.data_device = torch.from_numpy(batch.data).to("cuda:0")
    stream = torch.cuda.current_stream()

    def step():
        return ube.encode(model, arena, batch, completion=1, stream=stream)

    rows, stats = step()
    torch.cuda.synchronize()
    T = stats[1]
    if g["modality"] == "text":
        lengths = np.minimum(np.diff(batch.offsets.astype(np.int64)), g["context"])
        units = T  # encoded bytes
    else:
        per = (batch.heights // g["patch_side"]) * (batch.widths // g["patch_side"]) * batch.frames
        lengths = per.astype(np.int64)
        units = int(batch.data.size)  # pixel bytes
    flops = configs.encode_flops(g, lengths)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ube.kernel_timer_start(args.kernel, args.steps * g["depth"] + 8)
    torch.cuda.synchronize()
    ms, per = timed_steps(step, args.steps, stream)
    kms, launches = ube.kernel_timer_stop()

    per_kernel = {}
    if args.per_kernel:
        for kname in ube.KERNELS:
            ube.kernel_timer_start(kname, 4 * g["depth"] + 8)
            step()
            torch.cuda.synchronize()
            t, n = ube.kernel_timer_stop()
            if n:
                per_kernel[kname] = {"ms_per_step": t, "launches": n}

    kflops = kernel_flops_per_launch(args.kernel, g, T, lengths)
    avg_s = kms / max(launches, 1) / 1e3
    # E4M3 models run the block projections on fp8 MFMA (twice the bf16 rate); attention, the patch
    # projection and the pool stay bf16. Utilisation = the time at each precision's peak / the time taken.
    e4m3 = g["quantization"] == "e4m3"
    D, F = g["hidden"], g["ffn"]
    gemm_flops = g["depth"] * 2.0 * T * (D * 3 * D + D * D + D * 2 * F + F * D)
    fp8_flops = gemm_flops if e4m3 else 0.0
    ideal_s = fp8_flops / PEAK_FP8 + (flops - fp8_flops) / PEAK_BF16
    kpeak = PEAK_FP8 if (e4m3 and args.kernel.startswith("gemm_") and args.kernel != "gemm_patch") else PEAK_BF16
    traffic = load_traffic(args.kernel, args.workload)
    out = {
        "metric": METRIC,
        "value": units / (ms / 1e3),
        "unit": "bytes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        **step_stats(per),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if g["quantization"] == "e4m3" else "bf16",
        "data": "synthetic (seeded bytes, random-init bf16 weights N(0, 0.02))",
        "config": {"workload": f"{args.workload}: {WORKLOAD_TEXT[args.workload]}", "items": batch.count,
                   "tokens": int(T), "parallelism": "1 GPU"},
        "embeddings_per_s": batch.count / (ms / 1e3),
        "mfma_util": ideal_s / (ms / 1e3),
        "flops_per_step": flops,
        "fp8_flops_per_step": fp8_flops,
        "roofline": ({"kernel": args.kernel, "bound": "mfma", "achieved": kflops / avg_s / 1e12,
                      "peak": kpeak / 1e12, "unit": "TFLOP/s", "frac": kflops / avg_s / kpeak, "traffic": traffic,
                      "avg_launch_ms": avg_s * 1e3, "launches": launches} if kflops is not None else
                     {"kernel": args.kernel, "bound": "hbm",
                      "achieved": kernel_bytes_per_launch(args.kernel, g, T, batch.count) / avg_s / 1e9,
                      "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                      "frac": kernel_bytes_per_launch(args.kernel, g, T, batch.count) / avg_s / PEAK_HBM,
                      "traffic": traffic, "avg_launch_ms": avg_s * 1e3, "launches": launches}),
    }
    if per_kernel:
        out["per_kernel_ms"] = per_kernel
    if not args.no_cpu_baseline:
        default_rows = {"long": 1, "packed": 64, "image": 8, "video": 1, "video_e4m3": 1}.get(args.workload, 16)
        rows_s = ([int(r) for r in args.cpu_rows.split(",") if r != ""] if args.cpu_rows is not None
                  else list(range(min(default_rows, batch.count))))
        out["cpu_baseline"] = cpu_baseline(args.workload, weights, batch, rows_s)
    else:
        out["cpu_baseline"] = None
    arena.close()
    model.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
