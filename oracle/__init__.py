"""THE ORACLE -- test infrastructure only.

A plain fp64 CPU implementation of the decode step (see oracle.c for the arithmetic and its
citations) plus the bookkeeping around it: the per-layer K/V cache, greedy generation, the
recompute-from-scratch reference, and the expected status codes of every library entry point.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
It shares no code with the GPU library and never calls it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import contract  # noqa: F401  (re-exported)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, F64, Q8 = 0, 1, 2, 3
HALF_SPLIT, INTERLEAVED = 0, 1
_DT = {"f32": F32, "bf16": BF16, "f64": F64, "q8": Q8}


def build() -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp)."""
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp,
                           os.path.join(_HERE, "oracle.c"), "-lm"])
    os.replace(tmp, _SO)
    return _SO


class _Shape(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int64), ("d", ctypes.c_int64), ("n_layer", ctypes.c_int64),
                ("n_head", ctypes.c_int64), ("n_kv", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("hidden", ctypes.c_int64), ("eps", ctypes.c_double), ("rope_base", ctypes.c_double),
                ("rope_layout", ctypes.c_int32), ("w_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


_PP = ctypes.POINTER(ctypes.c_void_p)


class _Weights(ctypes.Structure):
    _fields_ = [("emb", ctypes.c_void_p), ("out", ctypes.c_void_p), ("norm", ctypes.c_void_p),
                ("wq", _PP), ("wk", _PP), ("wv", _PP), ("wo", _PP), ("gate", _PP), ("up", _PP),
                ("down", _PP), ("n1", _PP), ("n2", _PP)]


class _Cache(ctypes.Structure):
    _fields_ = [("k", _PP), ("v", _PP), ("max_seq", ctypes.c_int64)]


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        p, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "orc_gemv_t": ([p, i32, p, i64, i64, p], None),
            "orc_matvec": ([p, i32, p, i64, i64, p], None),
            "orc_rmsnorm": ([p, p, i64, f64, p], None),
            "orc_silu": ([f64], f64),
            "orc_rope": ([p, i64, i64, i64, f64, i32], None),
            "orc_attend": ([p, p, p, i32, i64, i64, i64, i64, p], None),
            "orc_argmax_f32": ([p, i64, p], i64),
            "orc_gemv_t_f32": ([p, i32, p, i64, i64, p], None),
            "orc_matvec_f32": ([p, i32, p, i64, i64, p], None),
            "orc_residual_add_f32": ([p, p, i64, p], None),
            "orc_add_rmsnorm_f32": ([p, p, p, i64, i64, f64, p], None),
            "orc_silu_mul_f32": ([p, p, i64, p], None),
            "orc_rope_f32": ([p, p, i64, i64, i64, i64, i64, f64, i32], None),
            "orc_rope_table_f32": ([i64, i64, f64, p], None),
            "orc_attend_f32": ([p, p, p, i32, i64, i64, i64, i64, p], None),
            "orc_kv_append_copy": ([p, i64, p, i64, i32, p], i64),
            "orc_forward_token": ([ctypes.POINTER(_Shape), ctypes.POINTER(_Weights), ctypes.POINTER(_Cache),
                                   i64, i64, p, p], ctypes.c_int),
            "orc_num_threads": ([], ctypes.c_int),
            "orc_bf16_to_double": ([ctypes.c_uint16], f64),
            "orc_widen": ([p, i32, i64, p], None),
            "orc_softmax_rows": ([p, i64, i64, p], None),
            "orc_silu_mul_inplace": ([p, p, i64], None),
            "orc_float_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
            "orc_q8_row": ([p, i64, p, ctypes.POINTER(ctypes.c_float)], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def _dtype_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float64:
        return F64
    raise TypeError(f"unsupported weight dtype {a.dtype}")


# ---------------------------------------------------------------------------------------------
# primitives (numpy in, numpy out)
# ---------------------------------------------------------------------------------------------

def gemv_t(a: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = A^T x in fp64 (A [m][n] of f32 / bf16-bits / f64)."""
    m, n = a.shape
    xd = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(n, dtype=np.float64)
    lib().orc_gemv_t(_ptr(a), _dtype_of(a), _ptr(xd), m, n, _ptr(y))
    return y


def gemv_t_f32(a: np.ndarray, x: np.ndarray) -> np.ndarray:
    m, n = a.shape
    xf = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(n, dtype=np.float32)
    lib().orc_gemv_t_f32(_ptr(a), _dtype_of(a), _ptr(xf), m, n, _ptr(y))
    return y


def matvec(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    rows, cols = w.shape
    xd = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty(rows, dtype=np.float64)
    lib().orc_matvec(_ptr(w), _dtype_of(w), _ptr(xd), rows, cols, _ptr(y))
    return y


def matvec_f32(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    rows, cols = w.shape
    xf = np.ascontiguousarray(x, dtype=np.float32)
    y = np.empty(rows, dtype=np.float32)
    lib().orc_matvec_f32(_ptr(w), _dtype_of(w), _ptr(xf), rows, cols, _ptr(y))
    return y


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float = 1e-5) -> np.ndarray:
    xd = np.ascontiguousarray(x, dtype=np.float64)
    gf = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty_like(xd)
    lib().orc_rmsnorm(_ptr(xd), _ptr(gf), xd.size, eps, _ptr(out))
    return out


def silu(z: float) -> float:
    return lib().orc_silu(float(z))


def rope(v: np.ndarray, n_heads: int, hd: int, pos: int, base: float, layout: int = HALF_SPLIT) -> np.ndarray:
    out = np.array(v, dtype=np.float64, copy=True)
    lib().orc_rope(_ptr(out), n_heads, hd, pos, base, layout)
    return out


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_head: int, n_kv: int, hd: int) -> np.ndarray:
    """q [n_head*hd] (fp64); k, v [ctx][n_kv][hd] of f32 / bf16-bits / f64."""
    qd = np.ascontiguousarray(q, dtype=np.float64)
    ctx = k.shape[0]
    out = np.empty(n_head * hd, dtype=np.float64)
    lib().orc_attend(_ptr(qd), _ptr(k), _ptr(v), _dtype_of(k), ctx, n_head, n_kv, hd, _ptr(out))
    return out


def attend_f32(q: np.ndarray, k: np.ndarray, v: np.ndarray, ctx: int, n_head: int, n_kv: int, hd: int) -> np.ndarray:
    qf = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty(n_head * hd, dtype=np.float32)
    lib().orc_attend_f32(_ptr(qf), _ptr(k), _ptr(v), _dtype_of(k), ctx, n_head, n_kv, hd, _ptr(out))
    return out


def argmax(logits: np.ndarray):
    """(token, value) of a 1-D fp32 row: first index of the maximum; first NaN if any."""
    lf = np.ascontiguousarray(logits, dtype=np.float32)
    best = ctypes.c_float()
    tok = lib().orc_argmax_f32(_ptr(lf), lf.size, ctypes.addressof(best))
    return int(tok), float(best.value)


def residual_add_f32(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    af, bf = np.ascontiguousarray(a, np.float32), np.ascontiguousarray(b, np.float32)
    out = np.empty_like(af)
    lib().orc_residual_add_f32(_ptr(af), _ptr(bf), af.size, _ptr(out))
    return out


def add_rmsnorm_f32(residual: np.ndarray, x, gain: np.ndarray, rows: int, n: int, eps: float):
    """Returns (residual_after, h)."""
    r = np.array(residual, dtype=np.float32, copy=True)
    h = np.empty_like(r)
    xs = None if x is None else np.ascontiguousarray(x, np.float32)
    g = np.ascontiguousarray(gain, np.float32)
    lib().orc_add_rmsnorm_f32(_ptr(r), None if xs is None else _ptr(xs), _ptr(g), rows, n, eps, _ptr(h))
    return r, h


def silu_mul_f32(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    g, u = np.ascontiguousarray(gate, np.float32), np.ascontiguousarray(up, np.float32)
    out = np.empty_like(g)
    lib().orc_silu_mul_f32(_ptr(g), _ptr(u), g.size, _ptr(out))
    return out


def rope_f32(q: np.ndarray, k, rows: int, n_q: int, n_k: int, hd: int, pos0: int, base: float, layout: int):
    qq = np.array(q, dtype=np.float32, copy=True)
    kk = None if k is None else np.array(k, dtype=np.float32, copy=True)
    lib().orc_rope_f32(_ptr(qq), None if kk is None else _ptr(kk), rows, n_q, n_k, hd, pos0, base, layout)
    return qq, kk


def rope_table_f32(max_pos: int, hd: int, base: float) -> np.ndarray:
    t = np.empty(max_pos * hd, dtype=np.float32)
    lib().orc_rope_table_f32(max_pos, hd, base, _ptr(t))
    return t


def kv_append_copy(cache: np.ndarray, new_vals: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """cache ++ new_vals (new values rounded to dtype); cache given in the storage dtype."""
    dt = _DT[dtype]
    npdt = {F32: np.float32, BF16: np.uint16}[dt]
    c = np.ascontiguousarray(cache, dtype=npdt)
    nv = np.ascontiguousarray(new_vals, dtype=np.float32)
    out = np.empty(c.size + nv.size, dtype=npdt)
    n = lib().orc_kv_append_copy(_ptr(c), c.size, _ptr(nv), nv.size, dt, _ptr(out))
    assert n == out.size
    return out


def widen(a: np.ndarray, out: np.ndarray | None = None) -> np.ndarray:
    """Stored fp32 values or bf16 bit patterns (uint16) widened to fp64 (exact), all host threads; into `out`
    (fp64, contiguous, a.size elements) when given."""
    src = np.ascontiguousarray(a)
    if out is None:
        out = np.empty(src.shape, dtype=np.float64)
    assert out.dtype == np.float64 and out.flags.c_contiguous and out.size == src.size
    lib().orc_widen(_ptr(src), _dtype_of(src), src.size, _ptr(out))
    return out.reshape(src.shape)


def softmax_rows(s: np.ndarray, last: np.ndarray) -> np.ndarray:
    """In place: each row of s [rows][cols] (fp64, contiguous) softmaxed over entries 0..last[row], the rest 0."""
    assert s.dtype == np.float64 and s.flags.c_contiguous
    la = np.ascontiguousarray(last, dtype=np.int64)
    lib().orc_softmax_rows(_ptr(s), s.shape[0], s.shape[1], _ptr(la))
    return s


def silu_mul_inplace(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """In place: g = silu(g) * u (fp64, contiguous, same shape)."""
    assert g.dtype == np.float64 and u.dtype == np.float64 and g.flags.c_contiguous and u.flags.c_contiguous
    lib().orc_silu_mul_inplace(_ptr(g), _ptr(u), g.size)
    return g


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    f = lib().orc_bf16_to_double
    return np.array([f(int(b)) for b in np.ravel(bits)], dtype=np.float64).reshape(np.shape(bits))


def f32_to_bf16(vals) -> np.ndarray:
    f = lib().orc_float_to_bf16
    return np.array([f(float(v)) for v in np.ravel(vals)], dtype=np.uint16).reshape(np.shape(vals))


# ---------------------------------------------------------------------------------------------
# the decode step
# ---------------------------------------------------------------------------------------------

class Model:
    """A decoder held for the oracle: a Shape-like object and the weight dict of synth.model /
    synth.page_draws ({emb, out, norm, layers: [{wq, wk, wv, wo, gate, up, down, n1, n2}]})."""

    def __init__(self, shape, W: dict):
        self.shape = shape
        self.W = W
        w_dt = _dtype_of(W["emb"])
        kv = _DT[shape.kv_dtype]
        self._shape = _Shape(shape.vocab, shape.d, shape.n_layer, shape.n_head, shape.n_kv, shape.head_dim,
                             shape.hidden, shape.eps, shape.rope_base, shape.rope_layout, w_dt, kv)
        L = W["layers"]

        def arr(name):
            for layer in L:
                assert layer[name].flags.c_contiguous
            return (ctypes.c_void_p * len(L))(*[layer[name].ctypes.data for layer in L])

        self._arrs = {n: arr(n) for n in ("wq", "wk", "wv", "wo", "gate", "up", "down", "n1", "n2")}
        a = self._arrs
        self._weights = _Weights(W["emb"].ctypes.data, W["out"].ctypes.data, W["norm"].ctypes.data,
                                 a["wq"], a["wk"], a["wv"], a["wo"], a["gate"], a["up"], a["down"], a["n1"], a["n2"])

    def new_cache(self, max_seq: int) -> "Cache":
        return Cache(self.shape, max_seq)

    def forward_token(self, token: int, pos: int, cache: "Cache", want_hidden: bool = False):
        """One step; returns (logits fp32 [V], hidden fp32 [L][d] or None). Writes K/V at pos."""
        s = self.shape
        logits = np.empty(s.vocab, dtype=np.float32)
        hidden = np.empty((s.n_layer, s.d), dtype=np.float32) if want_hidden else None
        rc = lib().orc_forward_token(ctypes.byref(self._shape), ctypes.byref(self._weights), ctypes.byref(cache._c),
                                     int(token), int(pos), _ptr(logits), None if hidden is None else _ptr(hidden))
        if rc != 0:
            raise ValueError(f"oracle forward_token refused token={token} pos={pos}")
        return logits, hidden


def q8_row(x):
    """(codes int8 [n], scale float32) of one K/V row in the int8 cache format (oracle.c: orc_q8_row)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    q = np.zeros(x.shape[0], dtype=np.int8)
    s = ctypes.c_float(0.0)
    lib().orc_q8_row(_ptr(x), x.shape[0], q.ctypes.data, ctypes.byref(s))
    return q, np.float32(s.value)


def q8_rows_value(codes, scales) -> np.ndarray:
    """What int8 rows stand for: codes [..., hd] times their row's scale [...], exact in fp64."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scales, dtype=np.float64)[..., None]


class Cache:
    """Per-layer K and V, each [max_seq][n_kv][hd] in the shape's K/V dtype ([fwd] KVCache). For the int8
    K/V dtype ("q8") each layer's K and V is one byte buffer, the codes [max_seq][n_kv][hd] followed by the
    fp32 scales [max_seq][n_kv]; codes(l, which) and scales(l, which) view its two parts."""

    def __init__(self, shape, max_seq: int):
        self.q8 = shape.kv_dtype == "q8"
        self._rows, self._hd, self._n_kv = max_seq * shape.n_kv, shape.head_dim, shape.n_kv
        if self.q8:
            nb = self._rows * shape.head_dim + 4 * self._rows
            self.k = [np.zeros(nb, dtype=np.uint8) for _ in range(shape.n_layer)]
            self.v = [np.zeros(nb, dtype=np.uint8) for _ in range(shape.n_layer)]
        else:
            npdt = {"f32": np.float32, "bf16": np.uint16}[shape.kv_dtype]
            self.k = [np.zeros((max_seq, shape.n_kv, shape.head_dim), dtype=npdt) for _ in range(shape.n_layer)]
            self.v = [np.zeros((max_seq, shape.n_kv, shape.head_dim), dtype=npdt) for _ in range(shape.n_layer)]
        self.length = 0
        self._kp = (ctypes.c_void_p * shape.n_layer)(*[a.ctypes.data for a in self.k])
        self._vp = (ctypes.c_void_p * shape.n_layer)(*[a.ctypes.data for a in self.v])
        self._c = _Cache(self._kp, self._vp, max_seq)

    def codes(self, l: int, which: str = "k") -> np.ndarray:
        """int8 cache: the codes of layer l's K or V, [max_seq][n_kv][hd] (a view)."""
        b = (self.k if which == "k" else self.v)[l]
        return b[:self._rows * self._hd].view(np.int8).reshape(-1, self._n_kv, self._hd)

    def scales(self, l: int, which: str = "k") -> np.ndarray:
        """int8 cache: the scales of layer l's K or V, [max_seq][n_kv] (a view)."""
        b = (self.k if which == "k" else self.v)[l]
        return b[self._rows * self._hd:].view(np.float32).reshape(-1, self._n_kv)

    def values(self, l: int, which: str, n: int) -> np.ndarray:
        """Positions 0..n-1 of layer l's K or V as the values the cache holds, fp64 [n][n_kv][hd]."""
        if self.q8:
            return q8_rows_value(self.codes(l, which)[:n], self.scales(l, which)[:n])
        return widen((self.k if which == "k" else self.v)[l][:n])

    def fill_prefix(self, prefix: list):
        """Load seeded K/V (synth.kv_prefix; for the int8 cache synth.kv_prefix_q8, per layer
        ((K codes, K scales), (V codes, V scales))) into positions 0..n-1."""
        if self.q8:
            n = prefix[0][0][0].shape[0]
            for l, ((kq, ks), (vq, vs)) in enumerate(prefix):
                self.codes(l, "k")[:n] = kq
                self.scales(l, "k")[:n] = ks
                self.codes(l, "v")[:n] = vq
                self.scales(l, "v")[:n] = vs
            self.length = n
            return
        n = prefix[0][0].shape[0]
        for l, (kk, vv) in enumerate(prefix):
            self.k[l][:n] = kk
            self.v[l][:n] = vv
        self.length = n


def generate(model: Model, prompt, n_new: int, max_seq: int, cache: Cache | None = None, want_hidden=False):
    """Prefill the prompt token by token, then n_new greedy steps ([fwd] "The code": generate).
    Returns (tokens, per-step logits list, per-step hidden list)."""
    c = cache if cache is not None else model.new_cache(max_seq)
    pos = c.length
    logits = None
    for t in prompt:
        logits, _ = model.forward_token(int(t), pos, c)
        pos += 1
    toks, all_logits, all_hidden = [], [], []
    for _ in range(n_new):
        tok, _ = argmax(logits)
        toks.append(tok)
        logits, hid = model.forward_token(tok, pos, c, want_hidden)
        all_logits.append(logits)
        all_hidden.append(hid)
        pos += 1
    c.length = pos
    return toks, all_logits, all_hidden


def recompute_generate(model: Model, prompt, n_new: int, max_seq: int):
    """The cache-free reference: every step re-runs the whole sequence through a fresh cache
    ([fwd] "The correctness test")."""
    seq = [int(t) for t in prompt]
    for _ in range(n_new):
        c = model.new_cache(max_seq)
        lg = None
        for pos, t in enumerate(seq):
            lg, _ = model.forward_token(t, pos, c)
        seq.append(argmax(lg)[0])
    return seq[len(prompt):]
