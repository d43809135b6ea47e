"""MI355X-native forward pass of the uniform byte encoder: a thin ctypes binding over libube.

Every step of the forward pass runs in libube's gfx950 HIP kernels (built in-tree
by ``multimodal_embeddings_amd.build``); this module only marshals arguments.
The raw C entry points keep their C names (``ube_text_encode`` ...); ``Model``,
``Arena`` and ``text_encode`` / ``image_encode_pixels`` / ``video_encode_frames``
wrap them for numpy / torch callers. There is no CPU fallback: without the built
library every call raises ``ExtensionMissing``.
"""
from __future__ import annotations

import ctypes as C
import os
import weakref

import numpy as np

from . import configs

HERE = os.path.dirname(os.path.abspath(__file__))
# UBE_LIBRARY may name another build of libube.so (A/B comparisons of kernel versions)
LIB_PATH = os.environ.get("UBE_LIBRARY") or os.path.join(HERE, "libube.so")


class ExtensionMissing(RuntimeError):
    pass


# ------------------------------------------------------------------ C structs (include/ube.h)

SZ = C.c_size_t
VP = C.c_void_p


class ube_outcome_t(C.Structure):
    _fields_ = [("status", C.c_int), ("message", C.c_char_p)]


class ube_tape_view_t(C.Structure):
    _fields_ = [("data", VP), ("offsets", C.POINTER(SZ)), ("count", SZ)]


class ube_rows_view_t(C.Structure):
    _fields_ = [("data", VP), ("count", SZ), ("columns", SZ), ("stride", SZ), ("scalar", C.c_int)]


class ube_rows_tape_view_t(C.Structure):
    _fields_ = [("data", VP), ("offsets", VP), ("count", SZ), ("rows", SZ), ("columns", SZ), ("stride", SZ),
                ("scalar", C.c_int)]


class ube_encode_stats_t(C.Structure):
    _fields_ = [("truncated", SZ), ("tokens", SZ)]


class ube_geometry_t(C.Structure):
    _fields_ = [(n, SZ) for n in ("depth", "hidden", "heads", "ffn", "vocab", "context", "rope_axes", "patch_side",
                                  "channels")] + [("rope_base", C.c_float), ("rms_epsilon", C.c_float),
                                                  ("quantization", C.c_int), ("token_width", SZ)]


class ube_weights_t(C.Structure):
    _fields_ = [("embed", VP), ("patch_proj", VP)] + [
        (n, C.POINTER(VP)) for n in ("w_qkv", "w_o", "w_gate", "w_up", "w_down", "attn_norm", "mlp_norm")] + [
        ("final_norm", VP), ("pool_query", VP), ("pool_wk", VP), ("pool_wv", VP), ("token_head", VP)]


class ube_model_init_t(C.Structure):
    _fields_ = [("model", C.POINTER(VP)), ("outcome", C.POINTER(ube_outcome_t)), ("device", C.c_int),
                ("geometry", ube_geometry_t), ("weights", C.POINTER(ube_weights_t))]


class ube_model_description_t(C.Structure):
    _fields_ = [(n, SZ) for n in ("dimensions", "context", "depth", "heads", "ffn", "rope_axes")] + [
        ("quantization", C.c_int), ("memory_usage", SZ), ("device", C.c_int), ("token_width", SZ)]


class ube_model_describe_t(C.Structure):
    _fields_ = [("model", VP), ("outcome", C.POINTER(ube_outcome_t)),
                ("description", C.POINTER(ube_model_description_t))]


class ube_arena_init_t(C.Structure):
    _fields_ = [("arena", C.POINTER(VP)), ("outcome", C.POINTER(ube_outcome_t)), ("device", C.c_int),
                ("capacity_limit", SZ)]


_ENCODE_HEAD = [("model", VP), ("arena", VP), ("stream", VP), ("outcome", C.POINTER(ube_outcome_t)),
                ("completion", C.c_int)]
_ENCODE_TAIL = [("outputs_scalar", C.c_int), ("embeddings", C.POINTER(ube_rows_view_t)),
                ("stats", C.POINTER(ube_encode_stats_t)), ("trace_residual", VP), ("outputs", C.c_uint),
                ("states", C.POINTER(ube_rows_tape_view_t)), ("token_vectors", C.POINTER(ube_rows_tape_view_t))]


class ube_text_encode_t(C.Structure):
    _fields_ = _ENCODE_HEAD + [("texts", ube_tape_view_t)] + _ENCODE_TAIL


class ube_image_encode_pixels_t(C.Structure):
    _fields_ = _ENCODE_HEAD + [("pixels", ube_tape_view_t), ("heights", C.POINTER(SZ)),
                               ("widths", C.POINTER(SZ))] + _ENCODE_TAIL


class ube_video_encode_frames_t(C.Structure):
    _fields_ = _ENCODE_HEAD + [("frames", ube_tape_view_t), ("frame_counts", C.POINTER(SZ)),
                               ("heights", C.POINTER(SZ)), ("widths", C.POINTER(SZ))] + _ENCODE_TAIL


class ube_maxsim_t(C.Structure):
    _fields_ = [("stream", VP), ("outcome", C.POINTER(ube_outcome_t)), ("device", C.c_int), ("completion", C.c_int),
                ("queries", ube_rows_tape_view_t), ("documents", ube_rows_tape_view_t), ("query_prefix", SZ),
                ("query_span", SZ), ("scores", VP), ("scores_stride", SZ)]


class ube_edges_view_t(C.Structure):
    _fields_ = [("offsets", C.POINTER(SZ)), ("ids", C.POINTER(C.c_uint32)), ("weights", C.POINTER(C.c_float))]


class ube_relations_view_t(C.Structure):
    _fields_ = [("attract", ube_edges_view_t), ("repel", ube_edges_view_t), ("ignore", ube_edges_view_t)]


class ube_contrastive_t(C.Structure):
    _fields_ = [("arena", VP), ("stream", VP), ("outcome", C.POINTER(ube_outcome_t)), ("completion", C.c_int),
                ("embeddings", ube_rows_view_t), ("anchor_begin", SZ), ("anchor_count", SZ),
                ("matryoshka_dimensions", C.POINTER(SZ)), ("matryoshka_dimensions_count", SZ),
                ("inverse_temperature", C.c_float), ("bias", C.c_float), ("negatives", C.c_int),
                ("ambient_repulsion_weight", C.c_float), ("pair_loss", C.c_int), ("relations", ube_relations_view_t),
                ("want_loss", C.c_int), ("scalars", VP), ("gradient", VP), ("gradient_stride", SZ)]


class ube_trainer_init_t(C.Structure):
    _fields_ = [("trainer", C.POINTER(VP)), ("outcome", C.POINTER(ube_outcome_t)), ("model", VP),
                ("weights", C.POINTER(ube_weights_t)), ("beta1", C.c_float), ("decay_rate", C.c_float),
                ("epsilon1", C.c_float), ("clip_threshold", C.c_float), ("activation_recomputation", C.c_int)]


class ube_trainer_forward_t(C.Structure):
    _fields_ = [("trainer", VP), ("arena", VP), ("stream", VP), ("outcome", C.POINTER(ube_outcome_t)),
                ("completion", C.c_int), ("texts", ube_tape_view_t), ("embeddings", C.POINTER(ube_rows_view_t)),
                ("stats", C.POINTER(ube_encode_stats_t))]


class ube_trainer_backward_t(C.Structure):
    _fields_ = [("trainer", VP), ("arena", VP), ("stream", VP), ("outcome", C.POINTER(ube_outcome_t)),
                ("completion", C.c_int), ("texts", ube_tape_view_t), ("d_embeddings", VP),
                ("d_embeddings_stride", SZ), ("stats", C.POINTER(ube_encode_stats_t)), ("after_forward", C.c_int)]


class ube_trainer_step_t(C.Structure):
    _fields_ = [("trainer", VP), ("stream", VP), ("outcome", C.POINTER(ube_outcome_t)), ("completion", C.c_int),
                ("learning_rate", C.c_float)]


class ube_trainer_tensor_t(C.Structure):
    _fields_ = [("name", C.c_char_p), ("layer", SZ), ("rows", SZ), ("cols", SZ), ("master", VP),
                ("master_scalar", C.c_int), ("gradient", VP)]


STATUS = {0: "success", 1: "invalid_argument", 2: "shape_mismatch", 3: "out_of_memory", 4: "device", 5: "contended",
          6: "unsupported", 7: "internal"}
SCALAR = {"unknown": 0, "u8": 1, "bf16": 2, "f32": 3, "e4m3": 4}
KERNELS = ["gather", "patchify", "rmsnorm", "gemm_patch", "gemm_qkv", "attention", "gemm_out", "gemm_gate_up",
           "gemm_down", "final_norm", "pool", "quantize", "contrastive_cells", "contrastive_rows",
           "contrastive_cols", "attention_bwd", "weight_grad"]
NEGATIVES = {"ambient": 0, "named": 1}
PAIR_LOSS = {"derived": 0, "balanced": 1, "ranked": 2, "sigmoid": 3}

# every symbol the headers declare, with ctypes signatures
_SIGNATURES = {
    "ube_model_init": ([C.POINTER(ube_model_init_t)], None),
    "ube_model_describe": ([C.POINTER(ube_model_describe_t)], None),
    "ube_model_free": ([VP], None),
    "ube_arena_init": ([C.POINTER(ube_arena_init_t)], None),
    "ube_arena_free": ([VP], None),
    "ube_arena_capacity": ([VP], SZ),
    "ube_text_encode": ([C.POINTER(ube_text_encode_t)], None),
    "ube_image_encode_pixels": ([C.POINTER(ube_image_encode_pixels_t)], None),
    "ube_video_encode_frames": ([C.POINTER(ube_video_encode_frames_t)], None),
    "ube_maxsim": ([C.POINTER(ube_maxsim_t)], None),
    "ube_contrastive": ([C.POINTER(ube_contrastive_t)], None),
    "ube_trainer_init": ([C.POINTER(ube_trainer_init_t)], None),
    "ube_trainer_forward": ([C.POINTER(ube_trainer_forward_t)], None),
    "ube_trainer_backward": ([C.POINTER(ube_trainer_backward_t)], None),
    "ube_trainer_step": ([C.POINTER(ube_trainer_step_t)], None),
    "ube_trainer_tensors": ([VP, C.POINTER(ube_trainer_tensor_t), SZ], SZ),
    "ube_trainer_free": ([VP], None),
    "ube_tape_plan": ([C.POINTER(SZ), SZ, SZ, VP, VP, C.POINTER(ube_encode_stats_t)], C.c_int),
    "ube_status_name": ([C.c_int], C.c_char_p),
    "ube_step_gemm": ([VP, VP, VP, SZ, SZ, SZ, VP], C.c_int),
    "ube_step_rmsnorm": ([VP, VP, VP, SZ, SZ, C.c_float, VP], C.c_int),
    "ube_step_attention": ([VP, VP, SZ, VP, SZ, VP, SZ, VP, SZ, SZ, VP], C.c_int),
    "ube_step_quantize_e4m3": ([VP, VP, VP, SZ, SZ, VP], C.c_int),
    "ube_step_gemm_e4m3": ([VP, C.c_float, VP, VP, VP, SZ, SZ, SZ, VP], C.c_int),
    "ube_step_attention_static": ([VP, VP, SZ, VP, SZ, VP, SZ, VP, SZ, SZ, VP], C.c_int),
    "ube_step_qkv_rotary": ([VP, VP, SZ, SZ, SZ, VP, SZ, C.c_float, SZ, VP, VP, SZ, VP], C.c_int),
    "ube_kernel_timer_start": ([C.c_int, SZ], C.c_int),
    "ube_kernel_timer_stop": ([C.POINTER(C.c_double), C.POINTER(SZ)], C.c_int),
    "ube_kernel_name": ([C.c_int], C.c_char_p),
}

_lib = None


def lib():
    """The loaded libube.so; raises ExtensionMissing when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ExtensionMissing(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                                   "(python -c 'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


class UbeError(RuntimeError):
    def __init__(self, status, message):
        self.status = STATUS.get(status, str(status))
        super().__init__(f"{self.status}: {message.decode() if isinstance(message, bytes) else message}")


def _check(outcome):
    if outcome.status != 0:
        raise UbeError(outcome.status, outcome.message or b"")


def _ptr(a):
    """Device or host address of a torch tensor or numpy array (None -> NULL)."""
    if a is None:
        return None
    if hasattr(a, "data_ptr"):
        return a.data_ptr()
    return a.ctypes.data


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------ model / arena


def _weights_struct(weights, g):
    """ube_weights_t over host copies of ``weights`` (bf16 bits and fp32 gains); returns it with the arrays
    that must outlive the call."""
    bits, f32 = weights.bits, weights.f32
    keep = []

    def host(a, dtype):
        arr = np.ascontiguousarray(a, dtype=dtype)
        keep.append(arr)
        return arr.ctypes.data

    def per_layer(name, table, dtype):
        arr = (VP * max(g["depth"], 1))(*[host(x, dtype) for x in table[name]])
        keep.append(arr)
        return arr

    w = ube_weights_t()
    if g["modality"] == "text":
        w.embed = host(bits["embed"], np.uint16)
    else:
        w.patch_proj = host(bits["patch_proj"], np.uint16)
    for name in ("w_qkv", "w_o", "w_gate", "w_up", "w_down"):
        setattr(w, name, per_layer(name, bits, np.uint16))
    for name in ("attn_norm", "mlp_norm"):
        setattr(w, name, per_layer(name, f32, np.float32))
    w.final_norm = host(f32["final_norm"], np.float32)
    w.pool_query = host(bits["pool_query"], np.uint16)
    w.pool_wk = host(bits["pool_wk"], np.uint16)
    w.pool_wv = host(bits["pool_wv"], np.uint16)
    if g.get("token_width"):
        w.token_head = host(bits["token_head"], np.uint16)
    return w, keep


class Model:
    """A model on one GPU, built from host weights (``synth.Weights`` or a dict of the same names)."""

    def __init__(self, weights, device: int = 0):
        g = configs.complete(weights.geometry)
        self.geometry = g
        w, keep = _weights_struct(weights, g)
        geo = ube_geometry_t(g["depth"], g["hidden"], g["heads"], g["ffn"], g["vocab"], g["context"], g["rope_axes"],
                             g["patch_side"], g["channels"], g["rope_base"], g["rms_epsilon"],
                             SCALAR[g["quantization"]], g.get("token_width", 0))
        handle = VP()
        outcome = ube_outcome_t()
        args = ube_model_init_t(C.pointer(handle), C.pointer(outcome), device, geo, C.pointer(w))
        lib().ube_model_init(C.byref(args))
        _check(outcome)
        self.handle = handle
        self.device = device
        del keep

    def describe(self):
        d = ube_model_description_t()
        outcome = ube_outcome_t()
        lib().ube_model_describe(C.byref(ube_model_describe_t(self.handle, C.pointer(outcome), C.pointer(d))))
        _check(outcome)
        return {f: getattr(d, f) for f, _ in ube_model_description_t._fields_}

    def close(self):
        if getattr(self, "handle", None):
            lib().ube_model_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Arena:
    def __init__(self, device: int = 0, capacity_limit: int = 0):
        handle = VP()
        outcome = ube_outcome_t()
        lib().ube_arena_init(C.byref(ube_arena_init_t(C.pointer(handle), C.pointer(outcome), device,
                                                      capacity_limit)))
        _check(outcome)
        self.handle = handle
        self.device = device

    @property
    def capacity(self):
        return lib().ube_arena_capacity(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            lib().ube_arena_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Rows:
    """A rows view in arena memory (device); ``tensor()`` copies it into a torch tensor."""

    def __init__(self, view: ube_rows_view_t, device: int):
        self.data = view.data
        self.count, self.columns, self.stride = view.count, view.columns, view.stride
        self.scalar = {v: k for k, v in SCALAR.items()}[view.scalar]
        self.device = device

    @property
    def __cuda_array_interface__(self):
        typestr = "<f4" if self.scalar == "f32" else "<u2"
        item = 4 if self.scalar == "f32" else 2
        return {"shape": (self.count, self.columns), "typestr": typestr, "data": (self.data or 0, False),
                "strides": (self.stride, item), "version": 2}

    def tensor(self):
        import torch
        if self.count == 0:
            dt = torch.float32 if self.scalar == "f32" else torch.int16
            return torch.zeros((0, self.columns), dtype=dt, device=f"cuda:{self.device}")
        t = torch.as_tensor(self, device=f"cuda:{self.device}").clone()
        return t if self.scalar == "f32" else t.view(torch.int16).view(torch.bfloat16)


class RowsTape:
    """A rows tape in device memory: item i owns rows offsets[i] .. offsets[i+1] of a [rows x columns] matrix."""

    def __init__(self, view: ube_rows_tape_view_t, device: int, keep=None):
        self.view = view
        self.data, self.offsets_ptr = view.data, view.offsets
        self.count, self.rows, self.columns, self.stride = view.count, view.rows, view.columns, view.stride
        self.scalar = {v: k for k, v in SCALAR.items()}[view.scalar]
        self.device = device
        self._keep = keep

    def tensor(self):
        """A torch copy of the rows, [rows x columns] (float32 or bfloat16)."""
        import torch
        item = 4 if self.scalar == "f32" else 2
        if self.rows == 0:
            dt = torch.float32 if self.scalar == "f32" else torch.bfloat16
            return torch.zeros((0, self.columns), dtype=dt, device=f"cuda:{self.device}")
        holder = type("_Cai", (), {"__cuda_array_interface__": {
            "shape": (self.rows, self.columns), "typestr": "<f4" if item == 4 else "<u2",
            "data": (self.data, False), "strides": (self.stride, item), "version": 2}})()
        t = torch.as_tensor(holder, device=f"cuda:{self.device}").clone()
        return t if item == 4 else t.view(torch.int16).view(torch.bfloat16)

    def offsets(self):
        """The count+1 offsets, copied to the host."""
        import torch
        holder = type("_Cai", (), {"__cuda_array_interface__": {
            "shape": (self.count + 1,), "typestr": "<u8", "data": (self.offsets_ptr, False), "version": 2}})()
        return torch.as_tensor(holder, device=f"cuda:{self.device}").cpu().numpy().copy()


def rows_tape(rows, offsets, device: int = 0):
    """A RowsTape over a torch bfloat16/float32 [rows x columns] tensor and a device uint64 offsets tensor."""
    import torch
    scalar = SCALAR["bf16"] if rows.dtype == torch.bfloat16 else SCALAR["f32"]
    view = ube_rows_tape_view_t(rows.data_ptr(), offsets.data_ptr(), offsets.numel() - 1, rows.shape[0],
                                rows.shape[1], rows.stride(0) * rows.element_size(), scalar)
    return RowsTape(view, device, keep=(rows, offsets))


OUTPUTS = {"embeddings": 1, "states": 2, "token_vectors": 4}


def _outputs_bits(outputs):
    if outputs is None:
        return 0
    if isinstance(outputs, int):
        return outputs
    bits = 0
    for name in outputs:
        bits |= OUTPUTS[name]
    return bits


def _finish(model, rows, states, vectors, stats, bits):
    if bits == 0:
        return Rows(rows, model.device), (stats.truncated, stats.tokens)
    emb = Rows(rows, model.device) if bits & 1 else None
    st = RowsTape(states, model.device) if bits & 2 else None
    tv = RowsTape(vectors, model.device) if bits & 4 else None
    return emb, st, tv, (stats.truncated, stats.tokens)


def maxsim(queries: RowsTape, documents: RowsTape, scores, *, prefix=0, span=0, stream=None, completion=0,
           device: int = 0):
    """Hard MaxSim scores of every (query, document) pair into ``scores`` (device float32 [nq x >= nd])."""
    outcome = ube_outcome_t()
    args = ube_maxsim_t(_stream_handle(stream), C.pointer(outcome), device, completion, queries.view,
                        documents.view, prefix, span, _ptr(scores), scores.stride(0) if scores.dim() == 2 else 0)
    lib().ube_maxsim(C.byref(args))
    _check(outcome)
    return scores


def _edges(edges, keep):
    """ube_edges_view_t over a (offsets, ids, weights-or-None) triple or an object with those attributes."""
    if edges is None:
        return ube_edges_view_t()
    if isinstance(edges, tuple):
        off, ids, w = edges
    else:
        off, ids, w = edges.offsets, edges.ids, edges.weights
    off = np.ascontiguousarray(off, dtype=np.uint64)
    ids = np.ascontiguousarray(ids, dtype=np.uint32)
    keep += [off, ids]
    wp = None
    if w is not None:
        w = np.ascontiguousarray(w, dtype=np.float32)
        keep.append(w)
        wp = w.ctypes.data_as(C.POINTER(C.c_float))
    return ube_edges_view_t(off.ctypes.data_as(C.POINTER(SZ)), ids.ctypes.data_as(C.POINTER(C.c_uint32)), wp)


def contrastive(arena: Arena, embeddings, scalars, *, anchor_begin=0, anchor_count=None, widths=None,
                inverse_temperature=10.0, bias=-10.0, negatives="ambient", ambient_weight=1.0, pair_loss="sigmoid",
                attract=None, repel=None, ignore=None, want_loss=True, gradient=None, stream=None, completion=0):
    """Matryoshka sigmoid contrastive loss over bf16 device rows ``embeddings`` [count x columns] (a torch
    bfloat16 tensor). ``scalars``: device float32 of at least 3 + widths entries (loss, d/dt, d/db, width
    losses); ``gradient``: optional device float32 [count x columns] receiving d loss / d embeddings.
    Edge sets are (offsets, ids, weights) triples over the anchors (host arrays)."""
    import torch
    count, columns = embeddings.shape
    if embeddings.dtype != torch.bfloat16:
        raise TypeError("embeddings must be bfloat16")
    anchor_count = count - anchor_begin if anchor_count is None else anchor_count
    keep = []
    wd = None
    if widths is not None:
        wd = np.ascontiguousarray(widths, dtype=np.uint64)
        keep.append(wd)
    view = ube_rows_view_t(_ptr(embeddings), count, columns, embeddings.stride(0) * 2, SCALAR["bf16"])
    rel = ube_relations_view_t(_edges(attract, keep), _edges(repel, keep), _edges(ignore, keep))
    outcome = ube_outcome_t()
    args = ube_contrastive_t(arena.handle, _stream_handle(stream), C.pointer(outcome), completion, view, anchor_begin,
                             anchor_count, wd.ctypes.data_as(C.POINTER(SZ)) if wd is not None else None,
                             len(wd) if wd is not None else 0, inverse_temperature, bias, NEGATIVES[negatives],
                             ambient_weight, PAIR_LOSS[pair_loss], rel, 1 if want_loss else 0, _ptr(scalars),
                             _ptr(gradient), gradient.stride(0) * 4 if gradient is not None else 0)
    lib().ube_contrastive(C.byref(args))
    _check(outcome)
    return scalars, gradient


class _DeviceArray:
    """__cuda_array_interface__ over raw device memory (torch.as_tensor turns it into a view).

    ``owner`` is the object whose memory this is: torch keeps this array alive as long as
    any tensor made from it, and the array keeps the owner alive, so the memory outlives
    every view unless the owner is closed explicitly (which the owner refuses while
    views exist)."""

    def __init__(self, ptr, shape, typestr, owner=None):
        self.owner = owner
        self.__cuda_array_interface__ = {"shape": tuple(shape), "typestr": typestr, "data": (ptr or 0, False),
                                         "version": 2}


class Trainer:
    """Training state of a text model on its GPU: bf16 masters (fp32 gains), fp32 gradients, Adafactor."""

    def __init__(self, model: Model, weights, *, beta1=0.0, decay_rate=0.0, epsilon1=0.0, clip_threshold=0.0,
                 activation_recomputation=False):
        w, keep = _weights_struct(weights, model.geometry)
        handle = VP()
        outcome = ube_outcome_t()
        args = ube_trainer_init_t(C.pointer(handle), C.pointer(outcome), model.handle, C.pointer(w), beta1,
                                  decay_rate, epsilon1, clip_threshold, 1 if activation_recomputation else 0)
        lib().ube_trainer_init(C.byref(args))
        _check(outcome)
        del keep
        self.handle = handle
        self.model = model
        self._views = weakref.WeakSet()

    def tensors(self):
        """[(name, layer, master view, gradient view)] as torch tensors over the trainer's device memory.
        Each view keeps the trainer alive; ``close()`` refuses while any view exists."""
        import torch
        n = lib().ube_trainer_tensors(self.handle, None, 0)
        arr = (ube_trainer_tensor_t * n)()
        lib().ube_trainer_tensors(self.handle, arr, n)
        dev = f"cuda:{self.model.device}"
        out = []

        def view(ptr, shape, typestr):
            a = _DeviceArray(ptr, shape, typestr, owner=self)
            self._views.add(a)
            return torch.as_tensor(a, device=dev)

        for t in arr:
            shape = (t.rows, t.cols) if t.cols else (t.rows,)
            if t.master_scalar == SCALAR["bf16"]:
                master = view(t.master, shape, "<i2").view(torch.bfloat16)
            else:
                master = view(t.master, shape, "<f4")
            grad = view(t.gradient, shape, "<f4")
            out.append((t.name.decode(), t.layer, master, grad))
        return out

    def forward(self, arena: Arena, data, offsets, *, stream=None, completion=0):
        """-> (Rows of fp32 pooled embeddings in the arena, (truncated, tokens)); keeps the activations that
        ``backward(..., after_forward=True)`` differentiates."""
        off = np.ascontiguousarray(offsets, dtype=np.uint64)
        tape = ube_tape_view_t(_ptr(data), off.ctypes.data_as(C.POINTER(SZ)), len(off) - 1)
        outcome, stats, rows = ube_outcome_t(), ube_encode_stats_t(), ube_rows_view_t()
        args = ube_trainer_forward_t(self.handle, arena.handle, _stream_handle(stream), C.pointer(outcome), completion,
                                     tape, C.pointer(rows), C.pointer(stats))
        lib().ube_trainer_forward(C.byref(args))
        _check(outcome)
        return Rows(rows, self.model.device), (stats.truncated, stats.tokens)

    def backward(self, arena, data, offsets, d_embeddings, *, stream=None, completion=0, after_forward=False):
        """Gradients of every parameter from d loss / d pooled rows: over the last ``forward`` with
        ``after_forward`` (arena, data and offsets unused), else after running that forward here."""
        if after_forward:
            tape, handle = ube_tape_view_t(None, None, 0), None
        else:
            off = np.ascontiguousarray(offsets, dtype=np.uint64)
            tape, handle = ube_tape_view_t(_ptr(data), off.ctypes.data_as(C.POINTER(SZ)), len(off) - 1), arena.handle
        outcome = ube_outcome_t()
        stats = ube_encode_stats_t()
        args = ube_trainer_backward_t(self.handle, handle, _stream_handle(stream), C.pointer(outcome), completion,
                                      tape, _ptr(d_embeddings), 0, C.pointer(stats), 1 if after_forward else 0)
        lib().ube_trainer_backward(C.byref(args))
        _check(outcome)
        return stats.truncated, stats.tokens

    def step(self, learning_rate, *, stream=None, completion=0):
        outcome = ube_outcome_t()
        args = ube_trainer_step_t(self.handle, _stream_handle(stream), C.pointer(outcome), completion, learning_rate)
        lib().ube_trainer_step(C.byref(args))
        _check(outcome)

    def close(self):
        if getattr(self, "handle", None):
            if len(getattr(self, "_views", ())):
                raise RuntimeError("tensors() views of this trainer are still alive; drop them before close()")
            lib().ube_trainer_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _tape(data, offsets):
    off = np.ascontiguousarray(offsets, dtype=np.uint64)
    return ube_tape_view_t(_ptr(data), off.ctypes.data_as(C.POINTER(SZ)), len(off) - 1), off


def text_encode(model: Model, arena: Arena, data, offsets, *, stream=None, outputs_scalar="f32", completion=0,
                trace=None, outputs=None):
    """-> (Rows, (truncated, tokens)); with ``outputs`` (names or bits) -> (embeddings Rows | None,
    states RowsTape | None, token vectors RowsTape | None, (truncated, tokens)).
    ``data``: torch uint8 tensor (device) or numpy (host)."""
    tape, off = _tape(data, offsets)
    rows, stats, outcome = ube_rows_view_t(), ube_encode_stats_t(), ube_outcome_t()
    states, vectors, bits = ube_rows_tape_view_t(), ube_rows_tape_view_t(), _outputs_bits(outputs)
    args = ube_text_encode_t(model.handle, arena.handle, _stream_handle(stream), C.pointer(outcome), completion,
                             tape, SCALAR[outputs_scalar], C.pointer(rows), C.pointer(stats), _ptr(trace), bits,
                             C.pointer(states), C.pointer(vectors))
    lib().ube_text_encode(C.byref(args))
    _check(outcome)
    return _finish(model, rows, states, vectors, stats, bits)


def image_encode_pixels(model: Model, arena: Arena, data, offsets, heights, widths, *, stream=None,
                        outputs_scalar="f32", completion=0, trace=None, outputs=None):
    tape, off = _tape(data, offsets)
    hh = np.ascontiguousarray(heights, dtype=np.uint64)
    ww = np.ascontiguousarray(widths, dtype=np.uint64)
    rows, stats, outcome = ube_rows_view_t(), ube_encode_stats_t(), ube_outcome_t()
    states, vectors, bits = ube_rows_tape_view_t(), ube_rows_tape_view_t(), _outputs_bits(outputs)
    args = ube_image_encode_pixels_t(model.handle, arena.handle, _stream_handle(stream), C.pointer(outcome),
                                     completion, tape, hh.ctypes.data_as(C.POINTER(SZ)),
                                     ww.ctypes.data_as(C.POINTER(SZ)), SCALAR[outputs_scalar], C.pointer(rows),
                                     C.pointer(stats), _ptr(trace), bits, C.pointer(states), C.pointer(vectors))
    lib().ube_image_encode_pixels(C.byref(args))
    _check(outcome)
    return _finish(model, rows, states, vectors, stats, bits)


def video_encode_frames(model: Model, arena: Arena, data, offsets, frame_counts, heights, widths, *, stream=None,
                        outputs_scalar="f32", completion=0, trace=None, outputs=None):
    tape, off = _tape(data, offsets)
    ff = np.ascontiguousarray(frame_counts, dtype=np.uint64)
    hh = np.ascontiguousarray(heights, dtype=np.uint64)
    ww = np.ascontiguousarray(widths, dtype=np.uint64)
    rows, stats, outcome = ube_rows_view_t(), ube_encode_stats_t(), ube_outcome_t()
    states, vectors, bits = ube_rows_tape_view_t(), ube_rows_tape_view_t(), _outputs_bits(outputs)
    args = ube_video_encode_frames_t(model.handle, arena.handle, _stream_handle(stream), C.pointer(outcome),
                                     completion, tape, ff.ctypes.data_as(C.POINTER(SZ)),
                                     hh.ctypes.data_as(C.POINTER(SZ)), ww.ctypes.data_as(C.POINTER(SZ)),
                                     SCALAR[outputs_scalar], C.pointer(rows), C.pointer(stats), _ptr(trace), bits,
                                     C.pointer(states), C.pointer(vectors))
    lib().ube_video_encode_frames(C.byref(args))
    _check(outcome)
    return _finish(model, rows, states, vectors, stats, bits)


def encode(model: Model, arena: Arena, batch, **kw):
    """Dispatch a synth batch to the verb of the model's modality."""
    m = model.geometry["modality"]
    if m == "text":
        return text_encode(model, arena, batch.data_device if hasattr(batch, "data_device") else batch.data,
                           batch.offsets, **kw)
    data = batch.data_device if hasattr(batch, "data_device") else batch.data
    if m == "image":
        return image_encode_pixels(model, arena, data, batch.offsets, batch.heights, batch.widths, **kw)
    return video_encode_frames(model, arena, data, batch.offsets, batch.frames, batch.heights, batch.widths, **kw)


def tape_plan(offsets, context):
    """Host-only bookkeeping through the library -> (lengths, cu, (truncated, tokens))."""
    off = np.ascontiguousarray(offsets, dtype=np.uint64)
    count = len(off) - 1
    lengths = np.zeros(max(count, 1), np.uint32)
    cu = np.zeros(count + 1, np.uint32)
    stats = ube_encode_stats_t()
    st = lib().ube_tape_plan(off.ctypes.data_as(C.POINTER(SZ)), count, context, lengths.ctypes.data,
                             cu.ctypes.data, C.byref(stats))
    if st != 0:
        raise UbeError(st, b"tape plan refused")
    return lengths[:count], cu, (stats.truncated, stats.tokens)


# ------------------------------------------------------------------ steps and timing (include/ube_steps.h)


def _step(st):
    if st != 0:
        raise UbeError(st, b"step refused")


def step_gemm(w, x, y, M, N, K, stream=None):
    _step(lib().ube_step_gemm(_ptr(w), _ptr(x), _ptr(y), M, N, K, _stream_handle(stream)))


def step_rmsnorm(x, gain, h, T, D, eps, stream=None):
    _step(lib().ube_step_rmsnorm(_ptr(x), _ptr(gain), _ptr(h), T, D, eps, _stream_handle(stream)))


def step_attention(q, k, ldqk, vt, ldvt, o, ldo, cu, heads, stream=None):
    cu = np.ascontiguousarray(cu, dtype=np.uint32)
    _step(lib().ube_step_attention(_ptr(q), _ptr(k), ldqk, _ptr(vt), ldvt, _ptr(o), ldo, cu.ctypes.data,
                                   len(cu) - 1, heads, _stream_handle(stream)))


def step_attention_static(q, k, ldqk, vt, ldvt, o, ldo, cu, heads, stream=None):
    """ube_step_attention_static: the attention step with its tile list in the library's fixed buffer."""
    cu = np.ascontiguousarray(cu, dtype=np.uint32)
    _step(lib().ube_step_attention_static(_ptr(q), _ptr(k), ldqk, _ptr(vt), ldvt, _ptr(o), ldo, cu.ctypes.data,
                                          len(cu) - 1, heads, _stream_handle(stream)))


def step_quantize_e4m3(x, codes, scales, T, W, stream=None):
    _step(lib().ube_step_quantize_e4m3(_ptr(x), _ptr(codes), _ptr(scales), T, W, _stream_handle(stream)))


def step_qkv_rotary(w, x, M, D, K, pos, rope_axes, rope_base, positions, qk, vt, ldvt, stream=None):
    """pos: host int16 [M x 4] (coordinates on axes 0..2); synchronous."""
    pos = np.ascontiguousarray(pos, dtype=np.int16)
    if pos.size < 4 * M:
        raise ValueError("pos must hold M x 4 coordinates")
    _step(lib().ube_step_qkv_rotary(_ptr(w), _ptr(x), M, D, K, pos.ctypes.data, rope_axes, rope_base, positions,
                                    _ptr(qk), _ptr(vt), ldvt, _stream_handle(stream)))


def step_gemm_e4m3(w, w_scale, x, x_scale, y, M, N, K, stream=None):
    _step(lib().ube_step_gemm_e4m3(_ptr(w), w_scale, _ptr(x), _ptr(x_scale), _ptr(y), M, N, K,
                                   _stream_handle(stream)))


def kernel_timer_start(kernel: str, max_launches: int):
    _step(lib().ube_kernel_timer_start(KERNELS.index(kernel), max_launches))


def kernel_timer_stop():
    ms, n = C.c_double(), SZ()
    _step(lib().ube_kernel_timer_stop(C.byref(ms), C.byref(n)))
    return ms.value, n.value
