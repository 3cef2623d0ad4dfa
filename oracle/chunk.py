"""THE ORACLE's chunked forward -- test infrastructure only (see the package docstring).

The decode step of the C oracle (`oracle.Model.forward_token`) applied to many rows at once, in fp64 numpy:
the same arithmetic, taken a layer at a time over all rows so that the weight products run as matrix
products (a library primitive) instead of one mat-vec per token. This is how the pages run a prompt: "Inside
the engine", section "1. CausalLM: the forward path", takes a chunk of prompt rows through each layer, and
decode is the one-row chunk of the same step; "The forward pass end to end", section "The code", defines
what every row computes (forward_token). Two forms:

  forward_chunk  rows of ONE sequence at consecutive positions (a prompt, or the tokens a decode run fed
                 itself, teacher-forced): every row's K/V is appended at its position before any row
                 attends, and row i attends positions 0..pos0 + i -- exactly what the token-by-token order
                 sees, because row i never reads a position after its own.
  forward_rows   one row each of MANY sequences (the batched decode step): every row attends its own
                 cached prefix plus its own new K/V.

Arithmetic (as the C oracle): fp64 from the exact stored inputs (bf16 and fp32 widen exactly), K/V rounded to
the cache dtype via fp32 (bf16 by round-to-nearest-even) where they are stored, logits and hidden states
rounded to fp32 on output. Only the order of the fp64 sums differs from the token-by-token oracle (matrix
products block their sums), a difference of a few fp64 ulps; the pins hold the two forms together.
"""
from __future__ import annotations

import numpy as np

from . import q8_rows_value, silu_mul_inplace, softmax_rows, widen

HALF_SPLIT, INTERLEAVED = 0, 1


def to_f64(a: np.ndarray) -> np.ndarray:
    """Stored values (bf16 bit patterns as uint16, fp32, fp64) widened to fp64, exactly."""
    if a.dtype in (np.uint16, np.float32):
        return widen(a)
    return np.asarray(a, dtype=np.float64)


def round_kv(v: np.ndarray, kv_dtype: str) -> np.ndarray:
    """fp64 values stored in the cache dtype: one rounding to fp32, then for bf16 round-to-nearest-even on
    the fp32 bits (a NaN stays a quiet NaN)."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if kv_dtype == "f32":
        return f
    u = f.view(np.uint32).astype(np.uint64)
    b = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        b[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return b


def quantize_kv(v: np.ndarray):
    """The int8 cache format (oracle.c, orc_q8_row) over every row of v [..., hd] at once: values rounded to
    fp32; per row s = max|x| / 127 and codes rint(x / s) clamped to [-127, 127], both divisions fp32 and ties
    to even; a zero row has s = 0 and codes 0. Returns (codes int8 [..., hd], scales float32 [...])."""
    x = np.asarray(v, dtype=np.float64).astype(np.float32)
    s = np.divide(np.max(np.abs(x), axis=-1), np.float32(127), dtype=np.float32)
    nz = s > 0
    den = np.where(nz, s, np.float32(1))[..., None]
    q = np.where(nz[..., None], np.rint(np.divide(x, den, dtype=np.float32)), np.float32(0))
    return np.clip(q, -127, 127).astype(np.int8), s.astype(np.float32)


def store_kv(cache, l: int, pos0: int, k: np.ndarray, v: np.ndarray) -> None:
    """Rows pos0.. of layer l's K and V ([T][n_kv][hd], fp64) into an oracle Cache in its dtype."""
    T = k.shape[0]
    if getattr(cache, "q8", False):
        for which, val in (("k", k), ("v", v)):
            codes, scales = quantize_kv(val)
            cache.codes(l, which)[pos0:pos0 + T] = codes
            cache.scales(l, which)[pos0:pos0 + T] = scales
        return
    kv_dtype = "f32" if cache.k[l].dtype == np.float32 else "bf16"
    cache.k[l][pos0:pos0 + T] = round_kv(k, kv_dtype)
    cache.v[l][pos0:pos0 + T] = round_kv(v, kv_dtype)


def cached_kv(cache, l: int, n: int):
    """Positions 0..n-1 of layer l's K and V as the values the cache holds (fp64)."""
    if getattr(cache, "q8", False):
        return cache.values(l, "k", n), cache.values(l, "v", n)
    return to_f64(cache.k[l][:n]), to_f64(cache.v[l][:n])


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Per row: x * (mean(x^2) + eps)^(-1/2) * g ("The code": rmsnorm, eps inside the mean)."""
    ms = np.sum(x * x, axis=-1, keepdims=True) / x.shape[-1]
    return x * (1.0 / np.sqrt(ms + eps)) * to_f64(g)


def rope(v: np.ndarray, positions: np.ndarray, base: float, layout: int) -> np.ndarray:
    """Rotate v [rows][heads][hd] in place, row r by positions[r]: pair j turned by pos * base^(-2j/hd), angles
    in fp64; half-split pairs (j, j + hd/2), interleaved pairs (2j, 2j + 1) ("decode-ops", "Method")."""
    hd = v.shape[-1]
    half = hd // 2
    j = np.arange(half, dtype=np.float64)
    inv = np.power(float(base), -(2.0 * j) / float(hd))
    theta = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]     # [rows][half]
    c, s = np.cos(theta)[:, None, :], np.sin(theta)[:, None, :]
    if layout == INTERLEAVED:
        a, b = v[..., 0::2].copy(), v[..., 1::2].copy()
        v[..., 0::2] = a * c - b * s
        v[..., 1::2] = a * s + b * c
    else:
        a, b = v[..., :half].copy(), v[..., half:].copy()
        v[..., :half] = a * c - b * s
        v[..., half:] = a * s + b * c
    return v


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_head: int, n_kv: int) -> np.ndarray:
    """One query row q [n_head][hd] over k, v [ctx][n_kv][hd] (fp64): head h reads K/V head h // (n_head / n_kv);
    scores q . k / sqrt(hd), softmax with the maximum subtracted, weighted sum of v ("The code")."""
    hd = q.shape[-1]
    group = n_head // n_kv
    out = np.empty((n_head, hd))
    for g in range(n_kv):
        qg = q[g * group:(g + 1) * group]                   # [group][hd]
        s = (qg @ k[:, g, :].T) / np.sqrt(float(hd))         # [group][ctx]
        s = np.exp(s - s.max(axis=1, keepdims=True))
        s /= s.sum(axis=1, keepdims=True)
        out[g * group:(g + 1) * group] = s @ v[:, g, :]
    return out


def attend_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_head: int, n_kv: int, last: np.ndarray) -> np.ndarray:
    """attend() for many query rows of one sequence at once: row i (q [T][n_head][hd]) sees positions
    0..last[i] of k, v [ctx][n_kv][hd] (fp64); the positions past last[i] get weight exp(-inf) = 0, so each
    row's softmax is over exactly its own context. Returns [T][n_head][hd]."""
    T, hd = q.shape[0], q.shape[-1]
    group = n_head // n_kv
    ctx = k.shape[0]
    out = np.empty((T, n_head, hd))
    last = np.asarray(last, dtype=np.int64)
    for g in range(n_kv):
        kg, vg = np.ascontiguousarray(k[:, g, :]), np.ascontiguousarray(v[:, g, :])
        for r0 in range(0, T, 256):
            r1 = min(T, r0 + 256)
            qg = q[r0:r1, g * group:(g + 1) * group, :].reshape(-1, hd)         # [(r1-r0) group][hd]
            sc = np.ascontiguousarray(qg @ kg.T / np.sqrt(float(hd)))            # [(r1-r0) group][ctx]
            softmax_rows(sc, np.repeat(last[r0:r1], group))
            out[r0:r1, g * group:(g + 1) * group] = (sc @ vg).reshape(r1 - r0, group, hd)
    return out


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


class Weights:
    """fp64 copies of a decoder's weights (the dict synth.model / synth.page_draws returns), made one layer at
    a time on request into buffers reused from layer to layer, so an 8B-shaped model never sits in fp64 all at
    once (and the host does not fault in fresh pages for every layer)."""

    def __init__(self, shape, W: dict):
        self.s, self.W = shape, W
        self._l = None
        self._buf = {}

    def _widen(self, key, a: np.ndarray) -> np.ndarray:
        b = self._buf.get(key)
        if b is None or b.size != a.size:
            b = self._buf[key] = np.empty(a.size, dtype=np.float64)
        return widen(a, b)

    def layer(self, l: int) -> dict:
        if self._l != l:
            self._cur = {k: self._widen(k, v) for k, v in self.W["layers"][l].items()}
            self._l = l
        return self._cur

    def release(self) -> None:
        self._l = None
        self._cur = None
        self._buf = {}

    def emb_rows(self, tokens) -> np.ndarray:
        return to_f64(self.W["emb"][np.asarray(tokens, dtype=np.int64)])

    def head(self, h: np.ndarray, rows_per_block: int = 8192) -> np.ndarray:
        """logits = h W_out^T, W_out [V][d] widened a block of vocabulary rows at a time."""
        out = self.W["out"]
        V = out.shape[0]
        lg = np.empty((h.shape[0], V))
        for r0 in range(0, V, rows_per_block):
            blk = out[r0:r0 + rows_per_block]
            lg[:, r0:r0 + blk.shape[0]] = h @ self._widen("head" if blk.shape[0] == rows_per_block else "tail", blk).T
        return lg


def _layer_tail(s, Wl: dict, x: np.ndarray, att: np.ndarray) -> None:
    """x += att Wo; x += (silu(h Wg) * (h Wu)) Wd with h = rmsnorm(x) g2, for every row (in place)."""
    x += att @ Wl["wo"]
    h = rmsnorm(x, Wl["n2"], s.eps)
    x += silu_mul_inplace(np.ascontiguousarray(h @ Wl["gate"]), np.ascontiguousarray(h @ Wl["up"])) @ Wl["down"]


def forward_chunk(shape, weights: Weights, tokens, pos0: int, cache, want_hidden: bool = True):
    """Rows tokens[i] at positions pos0 + i of the sequence whose K/V live in `cache` (an oracle.Cache, K/V
    [max_seq][n_kv][hd] in the cache dtype; positions before pos0 already filled). Writes every row's K/V,
    returns (logits fp32 [T][V], hidden fp32 [T][L][d] or None)."""
    s = shape
    T = len(tokens)
    pos = pos0 + np.arange(T)
    H, Hkv, hd = s.n_head, s.n_kv, s.head_dim
    x = weights.emb_rows(tokens)
    hidden = np.empty((T, s.n_layer, s.d), dtype=np.float32) if want_hidden else None
    for l in range(s.n_layer):
        Wl = weights.layer(l)
        h = rmsnorm(x, Wl["n1"], s.eps)
        q = rope((h @ Wl["wq"]).reshape(T, H, hd), pos, s.rope_base, s.rope_layout)
        k = rope((h @ Wl["wk"]).reshape(T, Hkv, hd), pos, s.rope_base, s.rope_layout)
        v = (h @ Wl["wv"]).reshape(T, Hkv, hd)
        store_kv(cache, l, pos0, k, v)
        kc, vc = cached_kv(cache, l, pos0 + T)
        att = attend_causal(q, kc, vc, H, Hkv, pos).reshape(T, H * hd)
        _layer_tail(s, Wl, x, att)
        if want_hidden:
            hidden[:, l] = x
    logits = weights.head(rmsnorm(x, weights.W["norm"], s.eps)).astype(np.float32)
    weights.release()
    cache.length = max(getattr(cache, "length", 0), pos0 + T)
    return logits, hidden


def attend_pieces(q: np.ndarray, pieces, n_head: int, n_kv: int) -> np.ndarray:
    """attend() for one query row over a context given as consecutive pieces [(K, V)], each HEAD-major
    [n_kv][n][hd] (stored dtype or fp64): the scores of all pieces form one softmax per head, and the output
    sums every piece's weighted values. Returns [n_head][hd] (fp64)."""
    hd = q.shape[-1]
    group = n_head // n_kv
    pieces = [(k if k.dtype == np.float64 else to_f64(k), v if v.dtype == np.float64 else to_f64(v))
              for k, v in pieces]
    ctx = sum(k.shape[1] for k, _ in pieces)
    sc = np.empty((n_head, ctx))
    for g in range(n_kv):
        qg, c0 = q[g * group:(g + 1) * group], 0
        for k, _ in pieces:
            m = k.shape[1]
            sc[g * group:(g + 1) * group, c0:c0 + m] = qg @ k[g].T
            c0 += m
    sc /= np.sqrt(float(hd))
    softmax_rows(sc, np.full(n_head, ctx - 1))
    out = np.zeros((n_head, hd))
    for g in range(n_kv):
        c0 = 0
        for _, v in pieces:
            m = v.shape[1]
            out[g * group:(g + 1) * group] += sc[g * group:(g + 1) * group, c0:c0 + m] @ v[g]
            c0 += m
    return out


def forward_rows(shape, weights: Weights, tokens, positions, prefix, want_hidden: bool = True, progress=None):
    """One decode step of B sequences: row b feeds tokens[b] at positions[b] and attends its own cached
    positions 0..positions[b] - 1, given by prefix(l, b) as a list of consecutive pieces [(K, V)] (each
    head-major [n_kv][n][hd], stored dtype or fp64, together positions[b] long), plus the K/V it appends. Returns (logits
    fp32 [B][V], hidden fp32 [B][L][d] or None, new K/V per layer as a list of (K [B][n_kv][hd], V [B][n_kv][hd])
    in the cache dtype; for the int8 cache ((K codes, K scales), (V codes, V scales))). progress(l), when given, is
    called after each layer."""
    s = shape
    B = len(tokens)
    pos = np.asarray(positions, dtype=np.int64)
    H, Hkv, hd = s.n_head, s.n_kv, s.head_dim
    x = weights.emb_rows(tokens)
    hidden = np.empty((B, s.n_layer, s.d), dtype=np.float32) if want_hidden else None
    new_kv = []
    for l in range(s.n_layer):
        Wl = weights.layer(l)
        h = rmsnorm(x, Wl["n1"], s.eps)
        q = rope((h @ Wl["wq"]).reshape(B, H, hd), pos, s.rope_base, s.rope_layout)
        k = rope((h @ Wl["wk"]).reshape(B, Hkv, hd), pos, s.rope_base, s.rope_layout)
        v = (h @ Wl["wv"]).reshape(B, Hkv, hd)
        if s.kv_dtype == "q8":
            kq, vq = quantize_kv(k), quantize_kv(v)
            new_kv.append((kq, vq))
            k, v = q8_rows_value(*kq), q8_rows_value(*vq)
        else:
            k, v = round_kv(k, s.kv_dtype), round_kv(v, s.kv_dtype)
            new_kv.append((k, v))
        att = np.empty((B, H * hd))
        for b in range(B):
            pieces = list(prefix(l, b))
            assert sum(pk.shape[1] for pk, _ in pieces) == pos[b]
            new = (k[b:b + 1].transpose(1, 0, 2), v[b:b + 1].transpose(1, 0, 2))
            att[b] = attend_pieces(q[b], pieces + [new], H, Hkv).ravel()
        _layer_tail(s, Wl, x, att)
        if want_hidden:
            hidden[:, l] = x
        if progress:
            progress(l)
    logits = weights.head(rmsnorm(x, weights.W["norm"], s.eps)).astype(np.float32)
    weights.release()
    return logits, hidden, new_kv
