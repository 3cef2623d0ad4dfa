"""Moving host weights and K/V into device memory in the library's layouts (marshalling only).

Weights come as a dict of numpy arrays: 'emb' and 'out' [vocab][d], 'norm' [d] (fp32), and 'layers', a
list of dicts with 'wq', 'wk', 'wv', 'wo', 'gate', 'up', 'down' in the [in][out] layout and 'n1', 'n2'
(fp32 gains). Weight arrays are float32, or uint16 holding bf16 bit patterns.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (BF16, F32, Q8, W_IN_OUT, W_OUT_IN, Config, KVPool, Model, check, decode_step, decode_steps,
               decode_workspace_bytes, kv_reserve, make_config, q8_pack_bytes, quantize_q8, rope_table_init,
               transpose, workspace)

_LAYER_MAP = (("wq", "wq"), ("wk", "wk"), ("wv", "wv"), ("wo", "wo"), ("gate", "w_gate"), ("up", "w_up"),
              ("down", "w_down"), ("n1", "g_attn"), ("n2", "g_ffn"))


def config_from(shape, w_layout=W_OUT_IN, step_path=0) -> Config:
    """llmk_config from any object with vocab, d, n_layer, n_head, n_kv, head_dim, hidden, max_seq, eps,
    rope_base, rope_layout, w_dtype ('f32'/'bf16'/'q8') and kv_dtype attributes. upload_model repacks the
    projections to match w_layout. step_path: 0 auto, 1 one kernel per operation, 2 persistent. 'q8' means
    int8 weight packs of bf16 weights (the projections and the head; the embedding table stays bf16)."""
    code = {"f32": F32, "bf16": BF16, "q8": Q8}
    return make_config(shape.vocab, shape.d, shape.n_layer, shape.n_head, shape.n_kv, shape.head_dim, shape.hidden,
                       shape.max_seq, shape.eps, shape.rope_base, shape.rope_layout, code[shape.w_dtype],
                       code[shape.kv_dtype], w_layout, step_path)


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """float32 -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor. Flattened."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        t = torch.from_numpy(a.reshape(-1))
    elif a.dtype == np.uint16:
        t = torch.from_numpy(a.reshape(-1).view(np.int16)).view(torch.bfloat16)
    elif a.dtype == np.int8:
        t = torch.from_numpy(a.reshape(-1))
    else:
        raise TypeError(f"weights must be float32 or bf16 bits (uint16), got {a.dtype}")
    return t.to(device)


def _q8_pack(a: torch.Tensor, rows: int, cols: int, stream=None) -> torch.Tensor:
    """Quantize an output-major device matrix into a fresh int8 weight pack (on the device)."""
    pack = torch.empty(q8_pack_bytes(rows, cols), dtype=torch.uint8, device=a.device)
    check(quantize_q8(a, rows, cols, pack, stream), "quantize_q8")
    return pack


def upload_model(cfg: Config, W: dict, device="cuda", stream=None) -> Model:
    """Device weights for cfg. With cfg.w_dtype Q8 the weights come in bf16 (uint16) and every projection and
    the output head are quantized on the device into int8 weight packs (output-major)."""
    q8 = cfg.w_dtype == Q8
    emb = to_device(W["emb"], device)
    out = to_device(W["out"], device)
    if q8:
        out = _q8_pack(out, cfg.vocab, cfg.d, stream)
    norm = to_device(np.asarray(W["norm"], dtype=np.float32), device)
    layers = []
    for L in W["layers"]:
        dev_layer = {}
        for src, dst in _LAYER_MAP:
            if src in ("n1", "n2"):
                dev_layer[dst] = to_device(np.asarray(L[src], np.float32), device)
                continue
            a = to_device(L[src], device)               # [in][out], as given
            if cfg.w_layout == W_OUT_IN:                # repack once, on the device, into [out][in]
                rows, cols = L[src].shape
                t = torch.empty_like(a)
                check(transpose(a, t, rows, cols, stream), "transpose")
                del a
                a = t
                if q8:
                    a = _q8_pack(a, cols, rows, stream)
            dev_layer[dst] = a
        layers.append(dev_layer)
    table = torch.empty(cfg.max_seq * cfg.head_dim, dtype=torch.float32, device=device)
    check(rope_table_init(table, cfg.max_seq, cfg.head_dim, cfg.rope_base, stream), "rope_table_init")
    return Model(cfg, emb, out, norm, table, layers)


def new_pool(cfg: Config, n_slots: int, capacity: int, device="cuda", block_tokens=None, n_blocks=None) -> KVPool:
    """A contiguous pool, or with block_tokens and n_blocks a paged one."""
    return KVPool(cfg.n_layer, n_slots, capacity, cfg.n_kv, cfg.head_dim, cfg.kv_dtype, device,
                  block_tokens=block_tokens, n_blocks=n_blocks)


def _reserve(pool: KVPool, slot: int, n: int) -> None:
    if pool.paged and n > 0:
        check(kv_reserve(pool, slot, 0, n), "kv_reserve")


def fill_prefix(pool: KVPool, slot: int, prefix: list) -> None:
    """Copy host K/V for positions 0..n-1 (per layer (K, V), each [n][n_kv][hd] in the pool dtype) into a
    slot (a paged pool reserves its blocks first) and record its length."""
    q8 = pool.dtype == Q8    # prefix per layer ((K codes, K scales), (V codes, V scales))
    n = (prefix[0][0][0] if q8 else prefix[0][0]).shape[0]
    _reserve(pool, slot, n)
    dv = pool.k[0].device
    for l, (kk, vv) in enumerate(prefix):
        for which, x in (("k", kk), ("v", vv)):
            if q8:
                val = (to_device(x[0], dv).view(n, pool.n_kv, pool.head_dim), to_device(x[1], dv).view(n, pool.n_kv))
            else:
                val = to_device(x, dv).view(n, pool.n_kv, pool.head_dim)
            pool.write_positions(l, slot, which, 0, val)
    pool.set_len(slot, n)


class Decoder:
    """One sequence slot of a pool driven through decode_step / decode_steps."""

    def __init__(self, cfg: Config, model: Model, pool: KVPool, device="cuda"):
        self.cfg, self.model, self.pool = cfg, model, pool
        nbytes = decode_workspace_bytes(cfg, 1)
        if nbytes < 0:
            raise ValueError(f"config refused: {-nbytes}")
        self.ws = workspace(nbytes, device)
        self.token_out = torch.zeros(1, dtype=torch.int32, device=device)

    def step(self, token: int, pos: int, slot: int = 0, logits=None, hidden=None) -> int:
        return decode_step(self.cfg, self.model, self.pool, slot, token, pos, self.token_out, self.ws, logits, hidden)

    def steps(self, token0: int, pos0: int, n: int, tokens_out, slot: int = 0) -> int:
        return decode_steps(self.cfg, self.model, self.pool, slot, token0, pos0, n, tokens_out, self.ws)


def upload_kv_source(source: list, device="cuda") -> list:
    """Per layer (K, V) host arrays [n][Hkv][hd] (pool dtype; int8: (codes [n][Hkv][hd], scales [n][Hkv])) ->
    device tensors of the same shape."""
    def up(x):
        if isinstance(x, tuple):
            return tuple(to_device(a, device).view(a.shape) for a in x)
        return to_device(x, device).view(x.shape)
    return [(up(kk), up(vv)) for kk, vv in source]


def fill_prefix_window(pool: KVPool, slot: int, source_dev: list, start: int, n: int) -> None:
    """Copy positions [start, start + n) of a device K/V source into positions 0..n-1 of a slot and record
    its length (device-to-device)."""
    _reserve(pool, slot, n)
    for l, (kk, vv) in enumerate(source_dev):
        if n > 0:
            for which, x in (("k", kk), ("v", vv)):
                val = tuple(a[start:start + n] for a in x) if isinstance(x, tuple) else x[start:start + n]
                pool.write_positions(l, slot, which, 0, val)
    pool.set_len(slot, n)


class BatchDecoder:
    """Several slots of a pool driven together through decode_step_batch / decode_steps_batch."""

    def __init__(self, cfg: Config, model: Model, pool: KVPool, batch: int, device="cuda"):
        from . import decode_step_batch, decode_steps_batch  # noqa: F401
        self.cfg, self.model, self.pool, self.batch = cfg, model, pool, batch
        nbytes = decode_workspace_bytes(cfg, batch)
        if nbytes < 0:
            raise ValueError(f"config refused for batch {batch}: {-nbytes}")
        self.ws = workspace(nbytes, device)
        self.tokens_out = torch.zeros(batch, dtype=torch.int32, device=device)

    def step(self, slots, tokens, pos, logits=None, hidden=None) -> int:
        from . import decode_step_batch
        return decode_step_batch(self.cfg, self.model, self.pool, slots, tokens, pos, self.tokens_out, self.ws,
                                 logits, hidden)

    def steps(self, slots, tokens0, pos0, n: int, tokens_out) -> int:
        from . import decode_steps_batch
        return decode_steps_batch(self.cfg, self.model, self.pool, slots, tokens0, pos0, n, tokens_out, self.ws)
