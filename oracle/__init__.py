"""CPU oracle of the uniform byte encoder's forward pass (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; the product package never imports
it. It shares no code with the HIP path. Arithmetic is float64 (see oracle.c
for the definitions and the readings of the documentation pages).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (portable x86-64-v3, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


class Geometry(C.Structure):
    _fields_ = [("depth", C.c_size_t), ("hidden", C.c_size_t), ("heads", C.c_size_t), ("ffn", C.c_size_t),
                ("rope_axes", C.c_int), ("rope_base", C.c_double), ("rms_epsilon", C.c_double), ("e4m3", C.c_int)]


class Block(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down")]


P = C.c_void_p
SZ = C.c_size_t


def _declare(L):
    L.oracle_tape_plan.argtypes = [P, SZ, SZ, P, P, P]
    L.oracle_tape_plan.restype = C.c_int
    L.oracle_embed_text.argtypes = [P, P, P, P, SZ, P, SZ, P, P]
    L.oracle_embed_patches.argtypes = [P, C.c_uint64, C.c_uint64, C.c_uint64, SZ, SZ, P, SZ, C.c_int, P, P]
    L.oracle_e4m3_round.argtypes = [C.c_double]
    L.oracle_e4m3_round.restype = C.c_double
    L.oracle_e4m3_qdq.argtypes = [P, P, SZ]
    L.oracle_bf16_round.argtypes = [C.c_double]
    L.oracle_bf16_round.restype = C.c_double
    L.oracle_rmsnorm.argtypes = [P, P, SZ, SZ, C.c_double, P]
    L.oracle_rope_axis_of.argtypes = [SZ, SZ, C.c_int]
    L.oracle_rope_axis_of.restype = C.c_int
    L.oracle_rope.argtypes = [P, P, SZ, SZ, SZ, C.c_int, C.c_double]
    L.oracle_attention.argtypes = [P, P, P, P, SZ, SZ, SZ, P]
    L.oracle_swiglu.argtypes = [P, SZ, SZ, SZ, P, P, P, P]
    L.oracle_block.argtypes = [C.POINTER(Geometry), C.POINTER(Block), P, P, P, SZ, SZ]
    L.oracle_pool.argtypes = [P, P, SZ, SZ, SZ, P, P, P, P]
    L.oracle_forward.argtypes = [C.POINTER(Geometry), P, P, P, P, P, P, P, P, SZ, P]
    L.oracle_forward_states.argtypes = [C.POINTER(Geometry), P, P, P, P, P, SZ, P, P]
    L.oracle_token_vectors.argtypes = [P, SZ, SZ, P, SZ, P]
    L.oracle_maxsim.argtypes = [P, P, SZ, P, P, SZ, SZ, SZ, SZ, P]
    L.oracle_matmul.argtypes = [P, SZ, SZ, P, SZ, P, C.c_int]
    L.oracle_e4m3_weights.argtypes = [P, SZ, P]
    L.oracle_set_tap.argtypes = [P]


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


# ----------------------------------------------------------------- steps


class OracleError(ValueError):
    pass


def tape_plan(offsets, context):
    """-> (lengths uint64[count], cu uint64[count+1], (truncated, tokens))."""
    off = np.ascontiguousarray(offsets, dtype=np.uint64)
    count = len(off) - 1
    lengths = np.zeros(max(count, 1), np.uint64)
    cu = np.zeros(count + 1, np.uint64)
    stats = np.zeros(2, np.uint64)
    rc = lib().oracle_tape_plan(_p(off), count, int(context), _p(lengths), _p(cu), _p(stats))
    if rc != 0:
        raise OracleError("offsets decrease")
    return lengths[:count], cu, (int(stats[0]), int(stats[1]))


def embed_text(data, offsets, lengths, cu, embed):
    data = np.ascontiguousarray(data, dtype=np.uint8)
    off = np.ascontiguousarray(offsets, dtype=np.uint64)
    lengths = np.ascontiguousarray(lengths, dtype=np.uint64)
    cu = np.ascontiguousarray(cu, dtype=np.uint64)
    E = _f32(embed)
    count = len(lengths)
    T, D = int(cu[-1]), E.shape[1]
    x = np.zeros((max(T, 1), D), np.float64)
    pos = np.zeros((max(T, 1), 3), np.int32)
    lib().oracle_embed_text(_p(data), _p(off), _p(lengths), _p(cu), count, _p(E), D, _p(x), _p(pos))
    return x[:T], pos[:T]


def embed_patches(pixels, frames, height, width, channels, patch, patch_proj, axes):
    px = np.ascontiguousarray(pixels, dtype=np.uint8)
    W = _f32(patch_proj)
    D = W.shape[1]
    T = int(frames) * (int(height) // patch) * (int(width) // patch)
    x = np.zeros((max(T, 1), D), np.float64)
    pos = np.zeros((max(T, 1), 3), np.int32)
    lib().oracle_embed_patches(_p(px), int(frames), int(height), int(width), channels, patch, _p(W), D, axes,
                               _p(x), _p(pos))
    return x[:T], pos[:T]


def e4m3_round(v: float) -> float:
    return lib().oracle_e4m3_round(float(v))


def bf16_round(v: float) -> float:
    return lib().oracle_bf16_round(float(v))


def e4m3_qdq(a):
    a = _f64(a)
    out = np.empty_like(a)
    lib().oracle_e4m3_qdq(_p(a), _p(out), a.size)
    return out


def rmsnorm(x, g, eps):
    x = _f64(x)
    g = _f32(g)
    T, D = x.shape
    out = np.empty_like(x)
    lib().oracle_rmsnorm(_p(x), _p(g), T, D, float(eps), _p(out))
    return out


def rope_axis_of(pair, d, axes):
    return lib().oracle_rope_axis_of(pair, d, axes)


def rope(v, pos, heads, d, axes, base):
    """v: [T x heads*d] float64 (copied), pos: [T x 3] int32."""
    v = _f64(v).copy()
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    lib().oracle_rope(_p(v), _p(pos), v.shape[0], heads, d, axes, float(base))
    return v


def attention(q, k, v, cu, heads, d):
    q, k, v = _f64(q), _f64(k), _f64(v)
    cu = np.ascontiguousarray(cu, dtype=np.uint64)
    out = np.zeros_like(q)
    lib().oracle_attention(_p(q), _p(k), _p(v), _p(cu), len(cu) - 1, heads, d, _p(out))
    return out


def swiglu(h, w_gate, w_up, w_down):
    h = _f64(h)
    T, D = h.shape
    F = w_gate.shape[1]
    Wg, Wu, Wd = _f32(w_gate), _f32(w_up), _f32(w_down)
    out = np.zeros((T, D), np.float64)
    lib().oracle_swiglu(_p(h), T, D, F, _p(Wg), _p(Wu), _p(Wd), _p(out))
    return out


def pool(xf, cu, heads, query, wk, wv):
    xf = _f64(xf)
    cu = np.ascontiguousarray(cu, dtype=np.uint64)
    count = len(cu) - 1
    D = xf.shape[1] if xf.ndim == 2 else len(query)
    if xf.size == 0:
        xf = np.zeros((1, D), np.float64)
    q, Wk, Wv = _f32(query), _f32(wk), _f32(wv)
    out = np.zeros((max(count, 1), D), np.float64)
    lib().oracle_pool(_p(xf), _p(cu), count, D, heads, _p(q), _p(Wk), _p(Wv), _p(out))
    return out[:count]


def matmul(x, w, e4m3=False):
    """One block product y = x W (W used as given); with ``e4m3`` the rows of x are quantised per row
    (amax / 448 scale each) as the E4M3 blocks do."""
    x = _f64(x)
    W = _f64(w)
    T, K = x.shape
    N = W.shape[1]
    y = np.zeros((max(T, 1), N), np.float64)
    if T:
        lib().oracle_matmul(_p(x), T, K, _p(W), N, _p(y), 1 if e4m3 else 0)
    return y[:T]


def e4m3_weights(w):
    """A block matrix as the E4M3 blocks use it: one quantise-dequantise over the whole tensor."""
    w32 = _f32(w)
    out = np.empty(w32.shape, np.float64)
    lib().oracle_e4m3_weights(_p(w32), w32.size, _p(out))
    return out


_TAP_FN = C.CFUNCTYPE(None, C.c_char_p, C.POINTER(C.c_double), C.c_size_t, C.c_size_t)


class Taps:
    """Context manager recording what the blocks observe: ``taps[name]`` is the list (one entry per
    block, in order) of float64 copies of that value -- GEMM inputs as the products read them
    (``qkv_in``, ``out_in``, ``mlp_in``, ``up_in``, ``down_in``), weights as used (``w_qkv``, ``w_o``,
    ``w_gate``, ``w_up``, ``w_down``) and stored activations (``q``, ``k``, ``v``, ``o``, ``a``)."""

    def __init__(self):
        self.taps = {}

        def record(name, data, rows, cols):
            a = np.ctypeslib.as_array(data, shape=(rows * cols,)).reshape(rows, cols).copy() if rows * cols else \
                np.zeros((rows, cols))
            self.taps.setdefault(name.decode(), []).append(a)

        self._fn = _TAP_FN(record)

    def __enter__(self):
        lib().oracle_set_tap(C.cast(self._fn, C.c_void_p))
        return self.taps

    def __exit__(self, *exc):
        lib().oracle_set_tap(None)
        return False


# ------------------------------------------------------------ whole encoder


def _geometry(g, e4m3=None):
    if e4m3 is None:
        e4m3 = g.get("quantization", "bf16") == "e4m3"
    return Geometry(g["depth"], g["hidden"], g["heads"], g["ffn"], g["rope_axes"], float(g["rope_base"]),
                    float(g["rms_epsilon"]), 1 if e4m3 else 0)


class _Blocks:
    """Keeps the float32 arrays alive while C reads them."""

    def __init__(self, weights):
        f = weights.f32
        n = weights.geometry["depth"]
        self.keep = []
        self.arr = (Block * max(n, 1))()
        for l in range(n):
            vals = []
            for name in ("attn_norm", "w_qkv", "w_o", "mlp_norm", "w_gate", "w_up", "w_down"):
                a = _f32(f[name][l])
                self.keep.append(a)
                vals.append(a.ctypes.data)
            self.arr[l] = Block(*vals)


def forward(weights, x0, pos, cu, e4m3=None):
    """Blocks + final norm + pool over frontend rows x0 [T x D] -> pooled [count x D]."""
    g = weights.geometry
    geo = _geometry(g, e4m3)
    blocks = _Blocks(weights)
    x0 = _f64(x0)
    if x0.size == 0:
        x0 = np.zeros((1, g["hidden"]), np.float64)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    if pos.size == 0:
        pos = np.zeros((1, 3), np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.uint64)
    count = len(cu) - 1
    fn, pq = _f32(weights.f32["final_norm"]), _f32(weights.f32["pool_query"])
    wk, wv = _f32(weights.f32["pool_wk"]), _f32(weights.f32["pool_wv"])
    out = np.zeros((max(count, 1), g["hidden"]), np.float64)
    lib().oracle_forward(C.byref(geo), C.cast(blocks.arr, C.c_void_p), _p(fn), _p(pq), _p(wk), _p(wv), _p(x0),
                         _p(pos), _p(cu), count, _p(out))
    return out[:count]


def forward_states(weights, x0, pos, cu, e4m3=None):
    """-> (x after the N blocks, final-norm states xf), both [T x D]."""
    g = weights.geometry
    geo = _geometry(g, e4m3)
    blocks = _Blocks(weights)
    x0 = _f64(x0)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    cu = np.ascontiguousarray(cu, dtype=np.uint64)
    T = int(cu[-1])
    x = np.zeros((max(T, 1), g["hidden"]), np.float64)
    xf = np.zeros_like(x)
    fn = _f32(weights.f32["final_norm"])
    lib().oracle_forward_states(C.byref(geo), C.cast(blocks.arr, C.c_void_p), _p(fn), _p(x0), _p(pos), _p(cu),
                                len(cu) - 1, _p(x), _p(xf))
    return x[:T], xf[:T]


def encode_text(weights, data, offsets):
    """Whole text encode -> (pooled [count x D] float64, (truncated, tokens))."""
    g = weights.geometry
    lengths, cu, stats = tape_plan(offsets, g["context"])
    x0, pos = embed_text(data, offsets, lengths, cu, weights.f32["embed"])
    return forward(weights, x0, pos, cu), stats


def media_frontend(weights, batch):
    """Patch rows and positions of every item of a MediaBatch -> (x0, pos, cu)."""
    g = weights.geometry
    p, ch = g["patch_side"], g["channels"]
    xs, ps, lens = [], [], []
    off = batch.offsets.astype(np.int64)
    for i in range(batch.count):
        H, W, Fr = int(batch.heights[i]), int(batch.widths[i]), int(batch.frames[i])
        if H % p or W % p:
            raise OracleError("image side is not a multiple of the patch side")
        n = Fr * (H // p) * (W // p)
        if n > g["context"]:
            raise OracleError("patch count exceeds the context")
        x, pos = embed_patches(batch.data[off[i]:off[i + 1]], Fr, H, W, ch, p, weights.f32["patch_proj"],
                               g["rope_axes"])
        xs.append(x)
        ps.append(pos)
        lens.append(n)
    cu = np.zeros(batch.count + 1, np.uint64)
    cu[1:] = np.cumsum(lens)
    D = g["hidden"]
    x0 = np.concatenate(xs) if xs else np.zeros((0, D))
    pos = np.concatenate(ps) if ps else np.zeros((0, 3), np.int32)
    return x0, pos, cu


def encode_media(weights, batch):
    x0, pos, cu = media_frontend(weights, batch)
    return forward(weights, x0, pos, cu), (0, int(cu[-1]))


# ------------------------------------------------------- per-token outputs


def token_vectors(xf, w):
    """Unit rows of xf W (token head) -> [T x width] float64."""
    xf = _f64(xf)
    T, D = xf.shape
    w = _f32(w)
    width = w.shape[1]
    out = np.zeros((max(T, 1), width), np.float64)
    if T:
        lib().oracle_token_vectors(_p(xf), T, D, _p(w), width, _p(out))
    return out[:T]


def maxsim(q, q_offsets, d, d_offsets, prefix=0, span=64):
    """Hard MaxSim scores [len(q_offsets)-1 x len(d_offsets)-1] float64."""
    q, d = _f64(q), _f64(d)
    qo = np.ascontiguousarray(q_offsets, dtype=np.uint64)
    do = np.ascontiguousarray(d_offsets, dtype=np.uint64)
    nq, nd = len(qo) - 1, len(do) - 1
    width = q.shape[1] if q.ndim == 2 else d.shape[1]
    if q.size == 0:
        q = np.zeros((1, width), np.float64)
    if d.size == 0:
        d = np.zeros((1, width), np.float64)
    out = np.zeros((max(nq, 1), max(nd, 1)), np.float64)
    if nq and nd:
        lib().oracle_maxsim(_p(q), _p(qo), nq, _p(d), _p(do), nd, width, prefix, span, _p(out))
    return out[:nq, :nd]

