"""Seeded synthetic inputs for the decode step (weights, K/V prefixes, token ids).

Input plumbing shared by the oracle side and the GPU side of the tests and the
benchmark. Nothing here computes any part of the decode step; it only draws
numbers and lays them out. Every array is a pure function of its seed, so the two
sides see identical bytes.

Weight layouts follow the decoder description of the Inference Academy page ("The
forward pass end to end"): the seven per-layer projections are handed over in the
transposed-GEMV layout A[in][out] (y = A^T x, the llmk page, section "A parallel path
for one frozen kernel's known-slow shape"), while the embedding table and the output
head are [vocab][d].
"""
from __future__ import annotations

import ctypes
import os
import random
import subprocess
from dataclasses import dataclass, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    """Compile the generator library with gcc (OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    tmp = _SO + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"])
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        lib = ctypes.CDLL(_SO)
        p = ctypes.c_void_p
        i64, u64, f64 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        lib.synth_normal_f32.argtypes = [p, i64, u64, u64, f64, f64]
        lib.synth_normal_bf16.argtypes = [p, i64, u64, u64, f64, f64]
        lib.synth_uniform_i64.argtypes = [p, i64, u64, u64, i64, i64]
        for f in (lib.synth_normal_f32, lib.synth_normal_bf16, lib.synth_uniform_i64):
            f.restype = None
        _lib = lib
    return _lib


def normal(shape, seed: int, stream: int, std: float = 1.0, dtype: str = "f32", mean: float = 0.0) -> np.ndarray:
    """Seeded normal draws. dtype 'f32' -> float32 array; 'bf16' -> uint16 array of bf16 bit patterns."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "f32":
        out = np.empty(shape, dtype=np.float32)
        lib.synth_normal_f32(out.ctypes.data, n, seed, stream, mean, std)
    elif dtype == "bf16":
        out = np.empty(shape, dtype=np.uint16)
        lib.synth_normal_bf16(out.ctypes.data, n, seed, stream, mean, std)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


def ints(shape, lo: int, hi: int, seed: int, stream: int) -> np.ndarray:
    """Seeded uniform integers in [lo, hi] (inclusive), int64."""
    lib = _load()
    out = np.empty(shape, dtype=np.int64)
    lib.synth_uniform_i64(out.ctypes.data, int(out.size), seed, stream, lo, hi)
    return out


def draws(shape, seed: int, stream: int) -> np.ndarray:
    """Seeded uniform draws in [0, 1) on the grid k / 2^24, float32 (every value exact in fp32 and fp64)."""
    return (ints(shape, 0, (1 << 24) - 1, seed, stream).astype(np.float64) / float(1 << 24)).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# Workload shapes
# ----------------------------------------------------------------------------------------------

ROPE_HALF_SPLIT = 0
ROPE_INTERLEAVED = 1


@dataclass(frozen=True)
class Shape:
    """A decoder shape: vocab V, width d, layers L, query heads H, K/V heads Hkv, head dim hd, FFN width F."""
    name: str
    vocab: int
    d: int
    n_layer: int
    n_head: int
    n_kv: int
    head_dim: int
    hidden: int
    max_seq: int
    eps: float
    rope_base: float
    rope_layout: int
    w_dtype: str       # 'f32' | 'bf16'
    kv_dtype: str      # 'f32' | 'bf16'
    w_std: float

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


# The Inference Academy page's toy decoder: vocab 40, d 16, 2 layers, 4 query heads over 2 K/V heads
# (head_dim 16 // 4 = 4), SwiGLU width 24, max_seq 64, eps 1e-5, RoPE base 1e4, weights N(0, 0.15).
TINY = Shape("tiny-llama fp32 (V40 d16 L2 H4/2 hd4 F24)", 40, 16, 2, 4, 2, 4, 24, 64, 1e-5, 1e4,
             ROPE_HALF_SPLIT, "f32", "f32", 0.15)
# Qwen3-0.6B-shaped: d 1024, 28 layers, 16/8 heads at head_dim 128, SwiGLU 3072, vocab 151,936, base 1e6.
Q06 = Shape("qwen3-0.6b-shaped bf16 (V151936 d1024 L28 H16/8 hd128 F3072)", 151936, 1024, 28, 16, 8, 128, 3072,
            2176, 1e-5, 1e6, ROPE_HALF_SPLIT, "bf16", "f32", 0.02)
# Llama-3-8B-shaped: d 4096, 32 layers, 32/8 heads at head_dim 128, SwiGLU 14,336, vocab 128,256, base 5e5.
L8B = Shape("llama-3-8b-shaped bf16 (V128256 d4096 L32 H32/8 hd128 F14336)", 128256, 4096, 32, 32, 8, 128, 14336,
            4352, 1e-5, 5e5, ROPE_HALF_SPLIT, "bf16", "bf16", 0.02)

LAYER_TENSORS = ("wq", "wk", "wv", "wo", "gate", "up", "down", "n1", "n2")


def layer_shapes(s: Shape) -> dict:
    """[in][out] shapes of the per-layer projections and the two norm gains."""
    qd, kvd = s.n_head * s.head_dim, s.n_kv * s.head_dim
    return {"wq": (s.d, qd), "wk": (s.d, kvd), "wv": (s.d, kvd), "wo": (qd, s.d),
            "gate": (s.d, s.hidden), "up": (s.d, s.hidden), "down": (s.hidden, s.d),
            "n1": (s.d,), "n2": (s.d,)}


def _stream_id(layer: int, name: str) -> int:
    if layer < 0:
        return {"emb": 0, "out": 1, "norm": 2}[name]
    return 16 + 16 * layer + LAYER_TENSORS.index(name)


def model(s: Shape, seed: int = 0) -> dict:
    """Seeded random-init weights of shape s: N(0, w_std) in s.w_dtype, unit norm gains (float32).

    Returns {'emb': [V][d], 'out': [V][d], 'norm': [d], 'layers': [{wq, wk, wv, wo, gate, up, down, n1, n2}]}.
    """
    W = {"emb": normal((s.vocab, s.d), seed, _stream_id(-1, "emb"), s.w_std, s.w_dtype),
         "out": normal((s.vocab, s.d), seed, _stream_id(-1, "out"), s.w_std, s.w_dtype),
         "norm": np.ones(s.d, dtype=np.float32), "layers": []}
    shp = layer_shapes(s)
    for l in range(s.n_layer):
        L = {}
        for name in LAYER_TENSORS:
            if name in ("n1", "n2"):
                L[name] = np.ones(shp[name], dtype=np.float32)
            else:
                L[name] = normal(shp[name], seed, _stream_id(l, name), s.w_std, s.w_dtype)
        W["layers"].append(L)
    return W


def page_draws(s: Shape, seed: int = 0, std: float = 0.15) -> dict:
    """The toy decoder's weights drawn exactly as the Inference Academy page draws them.

    One Python `random.Random(seed)` stream, `gauss(0, std)` per element, matrices filled row by row
    in their [out][in] form, in the order emb, out, then per layer wq, wk, wv, wo, gate, up, down; all
    norm gains 1.0 (page section "The code"). The draw order has to match the page for its printed
    tokens to be reproducible. Returned as float64 in this module's layouts (projections transposed to
    [in][out]).
    """
    rng = random.Random(seed)

    def draw(rows, cols):
        flat = [rng.gauss(0.0, std) for _ in range(rows * cols)]
        return np.asarray(flat, dtype=np.float64).reshape(rows, cols)

    qd, kvd = s.n_head * s.head_dim, s.n_kv * s.head_dim
    W = {"emb": draw(s.vocab, s.d), "out": draw(s.vocab, s.d), "norm": np.ones(s.d, dtype=np.float32), "layers": []}
    for _ in range(s.n_layer):
        outs_ins = {"wq": (qd, s.d), "wk": (kvd, s.d), "wv": (kvd, s.d), "wo": (s.d, qd),
                    "gate": (s.hidden, s.d), "up": (s.hidden, s.d), "down": (s.d, s.hidden)}
        L = {}
        for name in ("wq", "wk", "wv", "wo", "gate", "up", "down"):
            L[name] = np.ascontiguousarray(draw(*outs_ins[name]).T)   # [out][in] -> [in][out]
        L["n1"] = np.ones(s.d, dtype=np.float32)
        L["n2"] = np.ones(s.d, dtype=np.float32)
        W["layers"].append(L)
    return W


def as_f32(W: dict) -> dict:
    """Round a float64 weight set (page_draws) to float32 for the fp32 tiny configuration."""
    out = {"emb": W["emb"].astype(np.float32), "out": W["out"].astype(np.float32),
           "norm": W["norm"].astype(np.float32), "layers": []}
    for L in W["layers"]:
        out["layers"].append({k: v.astype(np.float32) for k, v in L.items()})
    return out


def kv_prefix(s: Shape, n_pos: int, seed: int = 2, slot: int = 0) -> list:
    """Seeded K/V for positions 0..n_pos-1 of one slot: per layer (K, V), each [n_pos][Hkv][hd] in s.kv_dtype.

    Used where a workload names a filled cache rather than a prompt (the 8B-shaped step at context 4096).
    Values N(0, 1).
    """
    out = []
    for l in range(s.n_layer):
        pair = []
        for w in range(2):
            stream = 1_000_000 + (slot * s.n_layer + l) * 2 + w
            pair.append(normal((n_pos, s.n_kv, s.head_dim), seed, stream, 1.0, s.kv_dtype))
        out.append(tuple(pair))
    return out


def kv_prefix_q8(s: Shape, n_pos: int, seed: int = 2) -> list:
    """Seeded int8 K/V for positions 0..n_pos-1 of every layer: per layer ((K codes, K scales), (V codes, V
    scales)), codes int8 [n][n_kv][hd] uniform in [-127, 127], scales float32 [n][n_kv] = 0.02 + 0.01 |N(0, 1)|
    (rows of about N(0, 1) magnitudes). Drawn directly as bytes, like the other inputs: nothing is quantized."""
    out = []
    for l in range(s.n_layer):
        pair = []
        for w in range(2):
            st = 2 * l + w
            q = ints((n_pos, s.n_kv, s.head_dim), -127, 127, seed, 4000 + st).astype(np.int8)
            sc = (0.02 + 0.01 * np.abs(normal((n_pos, s.n_kv), seed, 5000 + st))).astype(np.float32)
            pair.append((q, sc))
        out.append(tuple(pair))
    return out


def prompt(n: int, vocab: int, seed: int = 1, stream: int = 0) -> np.ndarray:
    """Seeded uniform token ids in [0, vocab)."""
    return ints((n,), 0, vocab - 1, seed, 2_000_000 + stream)


PAGE_PROMPT = (3, 14, 15, 9, 2, 6)   # the Inference Academy page's cache-vs-recompute prompt


def ragged_contexts(n: int, lo: int, hi: int, seed: int = 3) -> np.ndarray:
    """Seeded context lengths, uniform integers in [lo, hi], one per batch row."""
    return ints((n,), lo, hi, seed, 3_000_000)


# A batched pool of many long sequences is filled from one seeded source per layer: slot s's prefix of
# c_s positions is positions [SLOT_WINDOW_STRIDE * s, SLOT_WINDOW_STRIDE * s + c_s) of the source, so every
# slot holds different values without drawing (and storing on the host) every slot separately.
SLOT_WINDOW_STRIDE = 97


def slot_window(slot: int) -> int:
    """First source position of a slot's prefix."""
    return SLOT_WINDOW_STRIDE * slot
