"""THE ORACLE -- test infrastructure only: int8 weight packs (q8), quantizer and inverse, plain numpy.

The pages speak of int8 weights and q8_K packs on their decode paths ([xpu] "1. CausalLM: the forward path", its
per-layer and device-residency paragraphs; [llmk] "How this composes into a decode step"; [dops], its opening paragraph) without fixing
a format, so the format is this library's own and this module is its definition:

  * a [rows][K] projection, output-major (each row is the weights of one output), is cut along K into groups
    of GROUP = 128 consecutive inputs of one row;
  * a group keeps the fp32 scale s = max|w| / 127 and the int8 codes q = rint(w / s), clamped to [-127, 127];
    an all-zero group has s = 0 and q = 0. The divisions are fp32 (one correctly rounded operation each) and
    rint rounds half to even, so a code is decided in fp32, as the library's kernel decides it;
  * the weight the decode step uses is q * s (exact in fp64);
  * the pack stores all rows * K codes row-major, then all rows * (K / GROUP) scales row-major (fp32, little
    endian): rows * K * (1 + 4 / GROUP) bytes.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this module.
"""
from __future__ import annotations

import os

import numpy as np

GROUP = 128


def pack_bytes(rows: int, K: int) -> int:
    return rows * K + 4 * rows * (K // GROUP)


def quantize(w) -> tuple[np.ndarray, np.ndarray]:
    """Codes int8 [rows][K] and scales float32 [rows][K / GROUP] of a float32 matrix (bf16 widened exactly)."""
    w = np.asarray(w, dtype=np.float32)
    rows, K = w.shape
    if K % GROUP:
        raise ValueError(f"K = {K} is not a multiple of {GROUP}")
    g = w.reshape(rows, K // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    s = np.divide(amax, np.float32(127), dtype=np.float32)
    nz = s > 0
    den = np.where(nz, s, np.float32(1))[..., None]
    q = np.rint(np.divide(g, den, dtype=np.float32))
    q = np.where(nz[..., None], q, np.float32(0))
    q = np.clip(q, -127, 127).astype(np.int8)
    return q.reshape(rows, K), s.astype(np.float32)


def dequantize(q: np.ndarray, s: np.ndarray, dtype=np.float64) -> np.ndarray:
    """The weights the codes stand for: q * s of their group, [rows][K]; float64 (every product is exact) or
    float32 (each product rounded once)."""
    rows, K = q.shape
    g = q.reshape(rows, K // GROUP, GROUP).astype(dtype) * s.astype(dtype)[..., None]
    return g.reshape(rows, K)


def to_pack(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """The pack's bytes (uint8): codes row-major, then scales row-major as little-endian fp32."""
    return np.concatenate([np.ascontiguousarray(q).view(np.uint8).ravel(),
                           np.ascontiguousarray(s, dtype="<f4").view(np.uint8).ravel()])


def from_pack(buf: np.ndarray, rows: int, K: int) -> tuple[np.ndarray, np.ndarray]:
    buf = np.asarray(buf, dtype=np.uint8).ravel()
    if buf.size != pack_bytes(rows, K):
        raise ValueError("pack size does not match the shape")
    q = buf[:rows * K].view(np.int8).reshape(rows, K)
    s = buf[rows * K:].view("<f4").reshape(rows, K // GROUP).astype(np.float32)
    return q, s


def widen(a: np.ndarray) -> np.ndarray:
    """float32 values of a weight array (uint16 holds bf16 bit patterns: the high half of an fp32)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return np.left_shift(a.astype(np.uint32), 16).view(np.float32)
    return a.astype(np.float32)


_PROJ = ("wq", "wk", "wv", "wo", "gate", "up", "down")


def _quantized_io(w_io: np.ndarray, dt) -> np.ndarray:
    """A projection given [in][out], quantized per output row along `in`, as q * s in [in][out] (blocks of
    output rows on a thread pool; every block is independent)."""
    from concurrent.futures import ThreadPoolExecutor
    n_in, n_out = w_io.shape
    out = np.empty((n_in, n_out), dt)
    step = 512

    def block(r0):
        r1 = min(n_out, r0 + step)
        rows = np.ascontiguousarray(widen(w_io[:, r0:r1]).T)   # [r1 - r0][in]
        out[:, r0:r1] = dequantize(*quantize(rows), dt).T

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(block, range(0, n_out, step)))
    return out


def quantized_weights(W: dict, f64: bool = True) -> dict:
    """The decoder the q8 format describes, as a weight dict for oracle.Model: every projection (given
    [in][out], quantized along `in` per output row) and the output head ([vocab][d], along d) replaced by q * s;
    the embedding table stays as it is stored (bf16 in the q8 format) and the gains are fp32. float64 weights
    (exact), or float32 (q * s rounded once; 2^-24 relative) to halve the memory of large shapes."""
    dt = np.float64 if f64 else np.float32
    out = {"emb": widen(W["emb"]).astype(dt, copy=False), "norm": np.asarray(W["norm"], np.float32)}
    out["out"] = np.ascontiguousarray(_quantized_io(np.asarray(W["out"]).T, dt).T)
    layers = []
    for L in W["layers"]:
        M = {"n1": np.asarray(L["n1"], np.float32), "n2": np.asarray(L["n2"], np.float32)}
        for k in _PROJ:
            M[k] = _quantized_io(np.asarray(L[k]), dt)
        layers.append(M)
    out["layers"] = layers
    return out
