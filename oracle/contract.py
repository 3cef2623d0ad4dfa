"""THE ORACLE's status expectations -- test infrastructure only.

For every library entry point, the status code its arguments must produce, written
independently of the library from the llmk page's status vocabulary ("LLM inference
kernels", section "Status vocabulary and the shape checks (contract)") and its guarantees
(section "Guarantees": exact-length checks before any read, zero or negative dimensions
refused, n_new = 0 refused, every dimension bounded by 1 << 24).

Precedence when several checks fail: null pointer / unknown enum (578), dimension < 1
(561), dimension > MAX_DIM (564), buffer lengths in argument order, value ranges, workspace.
Pointers are modelled as booleans (True = non-null); workspace sizes are the library's
business, so these functions assume a sufficient workspace unless `ws_short` is given.
"""
from __future__ import annotations

MAX_DIM = 1 << 24

NAMES = {
    560: "llmk_ok",
    561: "llmk_empty_dimension",
    562: "llmk_a_length_mismatch",
    563: "llmk_b_length_mismatch",
    564: "llmk_dimension_too_large",
    565: "llmk_code_out_of_range",
    566: "llmk_cache_length_mismatch",
    567: "llmk_new_length_mismatch",
    568: "llmk_logits_length_mismatch",
    569: "llmk_gemv_a_length_mismatch",
    570: "llmk_gemv_x_length_mismatch",
    571: "llmk_cache_capacity_exceeded",
    572: "llmk_token_out_of_range",
    573: "llmk_position_out_of_range",
    574: "llmk_head_shape_invalid",
    575: "llmk_slot_out_of_range",
    576: "llmk_weight_length_mismatch",
    577: "llmk_output_length_mismatch",
    578: "llmk_invalid_argument",
    579: "llmk_device_error",
}
OK, EMPTY, A_LEN, B_LEN, TOO_LARGE, OUT_OF_RANGE = 560, 561, 562, 563, 564, 565
CACHE_LEN, NEW_LEN, LOGITS_LEN, GEMV_A, GEMV_X, CAPACITY = 566, 567, 568, 569, 570, 571
TOKEN, POSITION, HEAD_SHAPE, SLOT, WEIGHT_LEN, OUTPUT_LEN, INVALID, DEVICE = 572, 573, 574, 575, 576, 577, 578, 579


def status_name(code: int) -> str:
    return NAMES.get(int(code), NAMES[OUT_OF_RANGE])


def _dims(*dims, allow_zero=()):
    """561 / 564 over dimensions; indices in allow_zero may be 0 (but not negative)."""
    for i, v in enumerate(dims):
        if v < (0 if i in allow_zero else 1):
            return EMPTY
    for v in dims:
        if v > MAX_DIM:
            return TOO_LARGE
    return OK


# ---- the four contract checks -------------------------------------------------------------

def residual_dims_check(n, len_a, len_b):
    c = _dims(n)
    if c != OK:
        return c
    if len_a != n:
        return A_LEN
    if len_b != n:
        return B_LEN
    return OK


def kv_append_dims_check(cache_len, len_cache, n_new, len_new):
    c = _dims(cache_len, n_new, allow_zero=(0,))
    if c != OK:
        return c
    if len_cache != cache_len:
        return CACHE_LEN
    if len_new != n_new:
        return NEW_LEN
    return OK


def argmax_dims_check(n, len_logits):
    c = _dims(n)
    if c != OK:
        return c
    return LOGITS_LEN if len_logits != n else OK


def gemv_dims_check(m, n, len_a, len_x):
    c = _dims(m, n)
    if c != OK:
        return c
    if len_a != m * n:
        return GEMV_A
    if len_x != m:
        return GEMV_X
    return OK


# ---- entry points ----------------------------------------------------------------------------

def gemv_t(a=True, len_a=0, a_dtype=0, x=True, len_x=0, m=0, n=0, y=True, len_y=0, ws=True, ws_short=False):
    if not (a and x and y and ws) or a_dtype not in (0, 1):
        return INVALID
    c = gemv_dims_check(m, n, len_a, len_x)
    if c != OK:
        return c
    if len_y != n:
        return OUTPUT_LEN
    return INVALID if ws_short else OK


def gemv(w=True, len_w=0, w_dtype=0, x=True, len_x=0, rows=0, cols=0, y=True, len_y=0):
    if not (w and x and y) or w_dtype not in (0, 1):
        return INVALID
    c = _dims(rows, cols)
    if c != OK:
        return c
    if len_w != rows * cols:
        return GEMV_A
    if len_x != cols:
        return GEMV_X
    if len_y != rows:
        return OUTPUT_LEN
    return OK


def residual_add(a=True, len_a=0, b=True, len_b=0, n=0, out=True, len_out=0):
    if not (a and b and out):
        return INVALID
    c = residual_dims_check(n, len_a, len_b)
    if c != OK:
        return c
    return OUTPUT_LEN if len_out != n else OK


def add_rmsnorm(residual=True, len_r=0, x=True, len_x=0, gain=True, len_g=0, rows=0, n=0, eps=1e-5, h=True, len_h=0):
    import math
    if not (residual and gain and h) or not (eps > 0 and math.isfinite(eps)):
        return INVALID
    c = _dims(rows, n)
    if c != OK:
        return c
    if len_r != rows * n:
        return A_LEN
    if x and len_x != rows * n:
        return B_LEN
    if len_g != n:
        return WEIGHT_LEN
    if len_h != rows * n:
        return OUTPUT_LEN
    return OK


def silu_mul(gate=True, len_gate=0, up=True, len_up=0, n=0, out=True, len_out=0):
    if not (gate and up and out):
        return INVALID
    c = _dims(n)
    if c != OK:
        return c
    if len_gate != n:
        return A_LEN
    if len_up != n:
        return B_LEN
    return OUTPUT_LEN if len_out != n else OK


# Shape limits. Only two of them come from the pages: RoPE rotates pairs, so head_dim is even, and every
# query head reads one K/V head, so n_head is a multiple of n_kv ("The forward pass end to end", "The
# code"). The rest are the library's own, as its header documents them for status 574: head_dim at most
# 256, a power of two for attention and the decode step, and at most 8 query heads per K/V head (the
# attention kernels keep a group's heads in one workgroup). They are restated here so that the status of
# every call is predicted; they are limits of the implementation, not of the method.
LIB_MAX_HEAD_DIM = 256
LIB_MAX_GROUP = 8


def _head_dim_ok(hd):
    """RoPE needs pairs (an even head dimension); the library takes at most LIB_MAX_HEAD_DIM."""
    return hd % 2 == 0 and 2 <= hd <= LIB_MAX_HEAD_DIM


def _attn_shape_ok(n_head, n_kv, hd):
    """Whole query-head groups (the method); at most LIB_MAX_GROUP heads per group and a power-of-two head
    dimension in [2, LIB_MAX_HEAD_DIM] (the library's kernels)."""
    return (n_head % n_kv == 0 and n_head // n_kv <= LIB_MAX_GROUP and 2 <= hd <= LIB_MAX_HEAD_DIM
            and (hd & (hd - 1)) == 0)


def rope_table_init(table=True, len_table=0, max_pos=0, head_dim=0, base=1e4):
    import math
    if not table or not (math.isfinite(base) and base > 1.0):
        return INVALID
    c = _dims(max_pos, head_dim)
    if c != OK:
        return c
    if not _head_dim_ok(head_dim):
        return HEAD_SHAPE
    return OUTPUT_LEN if len_table != max_pos * head_dim else OK


def rope(q=True, len_q=0, k=True, len_k=0, rows=0, n_q_heads=0, n_k_heads=0, head_dim=0, pos=True, len_pos=0,
         table=True, len_table=0, max_pos=0, layout=0):
    """Positions are device values the host cannot see: only their count is checked."""
    if not q or not table or not pos or layout not in (0, 1) or (not k and n_k_heads > 0):
        return INVALID
    c = _dims(rows, n_q_heads, head_dim, max_pos, n_k_heads, allow_zero=(4,))
    if c != OK:
        return c
    if not _head_dim_ok(head_dim):
        return HEAD_SHAPE
    if len_q != rows * n_q_heads * head_dim:
        return A_LEN
    if len_k != rows * n_k_heads * head_dim:
        return B_LEN
    if len_table != max_pos * head_dim:
        return WEIGHT_LEN
    if len_pos != rows:
        return OUTPUT_LEN
    return OK


def kv_append_flat(cache=True, capacity=0, dtype=0, cache_len=0, len_cache=0, new_vals=True, len_new=0, n_new=0):
    if not (cache and new_vals) or dtype not in (0, 1):
        return INVALID
    c = _dims(capacity)
    if c != OK:
        return c
    c = kv_append_dims_check(cache_len, len_cache, n_new, len_new)
    if c != OK:
        return c
    if cache_len + n_new > capacity:
        return CAPACITY
    return OK


def gqa_attend_flat(q=True, len_q=0, k_cache=True, v_cache=True, len_cache=0, kv_dtype=0, ctx_len=0, n_head=0,
                    n_kv=0, head_dim=0, out=True, len_out=0, ws=True, ws_short=False):
    if not (q and k_cache and v_cache and out and ws) or kv_dtype not in (0, 1):
        return INVALID
    c = _dims(ctx_len, n_head, n_kv, head_dim)
    if c != OK:
        return c
    if not _attn_shape_ok(n_head, n_kv, head_dim):
        return HEAD_SHAPE
    if len_q != n_head * head_dim:
        return A_LEN
    if len_cache < ctx_len * n_kv * head_dim:
        return B_LEN
    if len_out != n_head * head_dim:
        return OUTPUT_LEN
    return INVALID if ws_short else OK


def _pool_fields(pool):
    """A pool descriptor's own fields: 578 (null k, v or slot_len array, dtype), 561, 564, 574 (an int8 pool
    whose head_dim is not a multiple of 16), then 578 again for a layer buffer that is null or not 16-byte
    aligned (pool["buffers"] False), then the pages when the pool has them (pool["pages"])."""
    if not pool.get("arrays", True) or pool.get("dtype", 0) not in (0, 1, 2):
        return INVALID
    c = _dims(pool["n_layer"], pool["n_slots"], pool["capacity"], pool["n_kv"], pool["head_dim"])
    if c != OK:
        return c
    if pool.get("dtype", 0) == 2 and pool["head_dim"] % 16:
        return HEAD_SHAPE   # int8 rows of whole 16-code loads
    if not pool.get("buffers", True):
        return INVALID
    return _pages_fields(pool) if pool.get("pages") else OK


def _pages_fields(pool):
    """Paged pool ("Inside the engine", "3. The K/V cache and the block store": fixed blocks of block_tokens
    positions): 578 for a null table / host table / refcount array (pages["arrays"] False), block_tokens not a
    power of two in [64, 65536] or max_blocks != ceil(capacity / block_tokens); 561 for n_blocks < 1; 564 for
    n_blocks or n_slots * max_blocks above MAX_DIM."""
    g = pool["pages"]
    bt = g["block_tokens"]
    if not g.get("arrays", True):
        return INVALID
    if bt < 64 or bt > 65536 or bt & (bt - 1):
        return INVALID
    if g["max_blocks"] != -(-pool["capacity"] // bt):
        return INVALID
    if g["n_blocks"] < 1:
        return EMPTY
    if g["n_blocks"] > MAX_DIM or pool["n_slots"] * g["max_blocks"] > MAX_DIM:
        return TOO_LARGE
    return OK


def _paged(pool):
    """A pool for the paged-only entry points: its fields, then 578 when it has no pages."""
    if pool is None:
        return INVALID
    c = _pool_fields(pool)
    if c != OK:
        return c
    return OK if pool.get("pages") else INVALID


def kv_reserve(pool=None, slot=0, pos_begin=0, pos_end=0, need=0, n_free=0, capturing=False):
    """Status of llmk_kv_reserve; need: the blocks the reservation takes (fresh and copied, the oracle block
    manager's count), n_free: the pool's free blocks, capturing: the stream is being captured."""
    c = _paged(pool)
    if c != OK:
        return c
    if pos_begin < 0 or pos_end <= pos_begin:
        return EMPTY
    if pos_end > MAX_DIM:
        return TOO_LARGE
    if not (0 <= slot < pool["n_slots"]):
        return SLOT
    if pos_end > pool["capacity"] or need > n_free:
        return CAPACITY
    return INVALID if (need > 0 and capturing) else OK


def kv_fork(pool=None, src=0, dst=1, n_pos=1, src_len=0, dst_len=0, dst_blocks=0, src_blocks_ok=True,
            capturing=False):
    """Status of llmk_kv_fork; src_len / dst_len: the slots' recorded positions, dst_blocks: blocks dst holds,
    src_blocks_ok: every one of src's first n_pos positions has a block."""
    c = _paged(pool)
    if c != OK:
        return c
    if src == dst:
        return INVALID
    if n_pos < 1:
        return EMPTY
    if n_pos > MAX_DIM:
        return TOO_LARGE
    if not (0 <= src < pool["n_slots"] and 0 <= dst < pool["n_slots"]):
        return SLOT
    if n_pos > src_len or dst_len != 0 or dst_blocks or not src_blocks_ok:
        return CACHE_LEN
    return INVALID if capturing else OK


def kv_release(pool=None, slot=0):
    """Status of llmk_kv_release."""
    c = _paged(pool)
    if c != OK:
        return c
    return OK if 0 <= slot < pool["n_slots"] else SLOT


def kv_admit(pool=None, n_uncached=0, admit=True, n_free=0):
    """(status, admit) of llmk_kv_admit: admit when the free blocks cover ceil(n_uncached / block_tokens) plus
    one block of headroom ("Inside the engine", "2. The scheduler: continuous batching", "Admission")."""
    if not admit:
        return INVALID, None
    c = _paged(pool)
    if c != OK:
        return c, None
    if n_uncached < 0:
        return EMPTY, None
    if n_uncached > MAX_DIM:
        return TOO_LARGE, None
    bt = pool["pages"]["block_tokens"]
    return OK, int(n_free >= -(-n_uncached // bt) + 1)


def kv_pool_init(pool=None):
    """Status of llmk_kv_pool_init; pool is a dict of the descriptor's fields (None: null pointer)."""
    if pool is None:
        return INVALID
    return _pool_fields(pool)


def kv_append(pool=None, layer=0, slot=0, which=0, cache_len=0, recorded=0, new_vals=True, len_new=0, n_new=0,
              need=0, n_free=0, capturing=False, row_of=None):
    """(status, new_len, elem_offset) of llmk_kv_append into buffer `which` of (layer, slot); `recorded` is
    the pool's fill record of that buffer. The slot's region is a flat cache of plane elements at
    slot * plane ("Inside the engine", "3. The K/V cache and the block store"); the append follows the
    flat cache's rule ("LLM inference kernels", "KV-cache growth and greedy argmax"). A paged pool first
    reserves the positions the elements fall in (need / n_free / capturing as for kv_reserve) and the offset is
    that of the first element through the table: row_of(position) is the position's cache row after it."""
    if not new_vals or pool is None:
        return INVALID, None, None
    c = _pool_fields(pool)
    if c != OK:
        return c, None, None
    if not pool.get("records", True) or which not in (0, 1) or pool.get("dtype", 0) == 2 \
            or not (0 <= layer < pool["n_layer"]):
        return INVALID, None, None
    if cache_len < 0 or n_new < 1:
        return EMPTY, None, None
    if cache_len > MAX_DIM or n_new > MAX_DIM:
        return TOO_LARGE, None, None
    if not (0 <= slot < pool["n_slots"]):
        return SLOT, None, None
    if cache_len != recorded:
        return CACHE_LEN, None, None
    if len_new != n_new:
        return NEW_LEN, None, None
    row = pool["n_kv"] * pool["head_dim"]
    plane = pool["capacity"] * row
    if cache_len + n_new > plane:
        return CAPACITY, None, None
    if pool.get("pages"):
        if need > n_free:
            return CAPACITY, None, None
        if need > 0 and capturing:
            return INVALID, None, None
        p0 = cache_len // row
        return OK, cache_len + n_new, (row_of(p0) * row + cache_len - p0 * row) if row_of else None
    return OK, cache_len + n_new, slot * plane + cache_len


def gqa_attend(q=True, len_q=0, pool=None, layer=0, slot=0, ctx_len=0, n_head=0, out=True, len_out=0, rec_k=None,
               rec_v=None, ws=True, ws_short=False, blocks_ok=True):
    """Status of llmk_gqa_attend over (layer, slot) of a pool; rec_k / rec_v: the pool's fill records of
    that slot's K and V buffers in elements (None: the pool keeps none); blocks_ok (paged pools): every
    position of [0, ctx_len) has a block."""
    if not (q and out and ws) or pool is None:
        return INVALID
    c = _pool_fields(pool)
    if c != OK:
        return c
    if not (0 <= layer < pool["n_layer"]):
        return INVALID
    c = _dims(ctx_len, n_head)
    if c != OK:
        return c
    if not (0 <= slot < pool["n_slots"]):
        return SLOT
    n_kv, hd = pool["n_kv"], pool["head_dim"]
    if not _attn_shape_ok(n_head, n_kv, hd):
        return HEAD_SHAPE
    if len_q != n_head * hd:
        return A_LEN
    if len_out != n_head * hd:
        return OUTPUT_LEN
    if ctx_len > pool["capacity"] or (pool.get("pages") and not blocks_ok):
        return POSITION
    need = ctx_len * n_kv * hd
    if (rec_k is not None and rec_k < need) or (rec_v is not None and rec_v < need):
        return CACHE_LEN
    return INVALID if ws_short else OK


def argmax(logits=True, len_logits=0, rows=0, n=0, token=True, ws=True, ws_short=False):
    if not (logits and token and ws):
        return INVALID
    c = _dims(rows, n)
    if c != OK:
        return c
    if len_logits != rows * n:
        return LOGITS_LEN
    return INVALID if ws_short else OK


SAMPLE_MAX_K = 1024   # survivors the GPU sampler holds (top-k after clamping to n; 1 at temperature 0)
SAMPLE_MAX_ROWS = 65535   # rows one sampler call takes


def sample(logits=True, len_logits=0, rows=0, n=0, temperature=1.0, top_k=0, top_p=1.0, u=True, len_u=0,
           token=True, ws_short=False):
    """ws_short: the call needs a workspace (llmk_sample_workspace_bytes > 0) and gets none or too little."""
    if not (logits and u and token):
        return INVALID
    c = _dims(rows, n)
    if c != OK:
        return c
    if len_logits != rows * n:
        return LOGITS_LEN
    if len_u != rows:
        return B_LEN
    if not (temperature >= 0.0) or not (0.0 < top_p <= 1.0):
        return INVALID
    k = 1 if temperature == 0.0 else (n if top_k <= 0 or top_k >= n else top_k)
    if k > SAMPLE_MAX_K or rows > SAMPLE_MAX_ROWS:
        return TOO_LARGE
    return INVALID if ws_short else OK


def kv_slot_offset(n_slots, capacity, n_kv, head_dim, slot, pos, kv_head, table=None, block_tokens=None):
    """(status, offset): offset = slot*plane + pos*n_kv*hd + kv_head*hd, plane = capacity*n_kv*hd
    (the pool layout of "Inside the engine", section "3. The K/V cache and the block store"); with a block
    table ([slot][block], -1: none), offset = (table[slot][pos // bt] * bt + pos % bt)*n_kv*hd + kv_head*hd."""
    if not (0 <= slot < n_slots):
        return SLOT, None
    if not (0 <= pos < capacity):
        return POSITION, None
    if not (0 <= kv_head < n_kv):
        return HEAD_SHAPE, None
    if table is not None:
        b = table[slot][pos // block_tokens]
        if b < 0:
            return POSITION, None
        return OK, (b * block_tokens + pos % block_tokens) * n_kv * head_dim + kv_head * head_dim
    plane = capacity * n_kv * head_dim
    return OK, slot * plane + pos * n_kv * head_dim + kv_head * head_dim


Q8_GROUP = 128


def q8_pack_bytes(rows, cols):
    """llmk_q8_pack_bytes: bytes of an int8 weight pack, or -1."""
    if rows < 1 or cols < 1 or rows > MAX_DIM or cols > MAX_DIM or cols % Q8_GROUP:
        return -1
    return rows * cols + 4 * rows * (cols // Q8_GROUP)


def quantize_q8(w=True, len_w=0, w_dtype=0, rows=0, cols=0, pack=True, len_pack=0, aligned=True):
    """Expected status of llmk_quantize_q8 (aligned: both buffers start on a 16-byte boundary)."""
    if not (w and pack) or w_dtype not in (0, 1):
        return INVALID
    c = _dims(rows, cols)
    if c != OK:
        return c
    if cols % Q8_GROUP:
        return HEAD_SHAPE
    if len_w != rows * cols:
        return WEIGHT_LEN
    if len_pack != q8_pack_bytes(rows, cols):
        return OUTPUT_LEN
    if not aligned:
        return INVALID
    return OK


def config_check(vocab, d, n_layer, n_head, n_kv, head_dim, hidden, max_seq, eps=1e-5, rope_base=1e4, rope_layout=0,
                 w_dtype=0, kv_dtype=0, w_layout=0, step_path=0, test_flags=0):
    import math
    if rope_layout not in (0, 1) or w_dtype not in (0, 1, 2) or kv_dtype not in (0, 1, 2) or w_layout not in (0, 1):
        return INVALID
    if step_path not in (0, 1, 2) or test_flags not in (0, 1):
        return INVALID
    if not (eps > 0 and math.isfinite(eps)) or not (rope_base > 1 and math.isfinite(rope_base)):
        return INVALID
    c = _dims(vocab, d, n_layer, n_head, n_kv, head_dim, hidden, max_seq)
    if c != OK:
        return c
    if not _attn_shape_ok(n_head, n_kv, head_dim):
        return HEAD_SHAPE
    if kv_dtype == 2 and head_dim % 16:
        return HEAD_SHAPE   # the int8 cache's rows are whole loads of 16 codes
    if kv_dtype == 2 and step_path == 2:
        return INVALID      # the int8 cache runs one kernel per operation
    if w_dtype == 2:
        # int8 packs: projection inputs in whole groups of 128, at most 4 loads of 16 codes x 64 lanes per wave
        # over the widest split that leaves a wave 1,024 codes or more
        for k in (d, n_head * head_dim, hidden):
            kw = 4 if k // 4 >= 1024 else 2 if k // 2 >= 1024 else 1
            if k % Q8_GROUP or -(-(k // kw) // 1024) > 4:
                return HEAD_SHAPE
        if w_layout != 1:
            return INVALID
        return OK
    vec = 4 if w_dtype == 0 else 8
    for width in (d, n_head * head_dim, n_kv * head_dim, hidden):
        if width % vec != 0:
            return HEAD_SHAPE
    if d > 64 * vec * 16:
        return HEAD_SHAPE
    if w_layout == 1:
        # output-major projections: an input row of K elements is split over at most 4 waves, each holding
        # at most 8 vectors of 64 lanes x vec elements
        for k in (d, n_head * head_dim, hidden):
            if not any((k // kw) % vec == 0 and k % kw == 0 and -(-(k // kw) // (64 * vec)) <= 8 for kw in (1, 2, 4)):
                return HEAD_SHAPE
    if step_path == 2 and (w_dtype != 1 or w_layout != 1):
        return INVALID    # the persistent step runs bf16 output-major weights only
    return OK


def decode_step(cfg: dict, tensors_ok=True, lens_ok=True, pool_ok=True, pool_dims_bad=False, n_slots=1,
                capacity=0, slot=0, slot_len=0, token=0, pos=0, n_steps=1, logits=False, len_logits=0, hidden=False,
                len_hidden=0, ws_short=False):
    """Expected status of llmk_decode_step (n_steps = 1) and llmk_decode_steps. cfg holds config_check's
    arguments; tensors_ok / lens_ok say whether every model tensor is non-null / has the length the config
    implies; pool_ok whether the pool matches the config; pool_dims_bad whether n_slots or capacity < 1."""
    c = config_check(**cfg)
    if c != OK:
        return c
    if n_steps < 1:
        return EMPTY
    if n_steps > MAX_DIM:
        return TOO_LARGE
    if not tensors_ok:
        return INVALID
    if not lens_ok:
        return WEIGHT_LEN
    if not pool_ok:
        return INVALID
    if pool_dims_bad:
        return EMPTY
    if not (0 <= slot < n_slots):
        return SLOT
    if not (0 <= token < cfg["vocab"]):
        return TOKEN
    if pos < 0 or pos + n_steps > cfg["max_seq"]:
        return POSITION
    if pos != slot_len:
        return CACHE_LEN
    if pos + n_steps > capacity:
        return CAPACITY
    if logits and len_logits != cfg["vocab"]:
        return LOGITS_LEN
    if hidden and len_hidden != cfg["n_layer"] * cfg["d"]:
        return OUTPUT_LEN
    return INVALID if ws_short else OK


def decode_steps_sampled(cfg: dict, draws=True, len_draws=None, n_steps=1, temperature=1.0, top_k=0, top_p=1.0,
                         sample_ws_short=False, **step_kw):
    """Expected status of llmk_decode_steps_sampled: llmk_decode_steps' checks (decode_step's keywords, with
    n_steps), then the sampling arguments in llmk_sample's order."""
    if not draws:
        return INVALID
    ws_short = step_kw.pop("ws_short", False)   # the decode workspace is checked last
    c = decode_step(cfg, n_steps=n_steps, **step_kw)
    if c != OK:
        return c
    if (n_steps if len_draws is None else len_draws) != n_steps:
        return B_LEN
    if not (temperature >= 0.0) or not (0.0 < top_p <= 1.0):
        return INVALID
    n = cfg["vocab"]
    k = 1 if temperature == 0.0 else (n if top_k <= 0 or top_k >= n else top_k)
    if k > SAMPLE_MAX_K:
        return TOO_LARGE
    return INVALID if sample_ws_short or ws_short else OK


def decode_step_batch(cfg: dict, batch=1, tensors_ok=True, lens_ok=True, pool_ok=True, pool_dims_bad=False,
                      batch_weights_ok=True, n_slots=1, capacity=0, slots=(0,), slot_lens=None, tokens=(0,),
                      pos=(0,), n_steps=1, logits=False, len_logits=0, len_tokens=None, hidden=False, len_hidden=0,
                      ws_short=False):
    """Expected status of llmk_decode_step_batch (n_steps = 1) and llmk_decode_steps_batch (logits=False,
    hidden=False, len_tokens = n_steps * batch expected). slot_lens maps slot -> recorded length (default 0).
    batch_weights_ok: the weights are bf16 in the output-major layout the batched path runs on."""
    c = config_check(**cfg)
    if c != OK:
        return c
    if n_steps < 1:
        return EMPTY
    if n_steps > MAX_DIM:
        return TOO_LARGE
    if batch < 1:
        return EMPTY
    if batch > 64:
        return TOO_LARGE
    if not tensors_ok:
        return INVALID
    if not lens_ok:
        return WEIGHT_LEN
    if not pool_ok:
        return INVALID
    if pool_dims_bad:
        return EMPTY
    if not batch_weights_ok:
        return INVALID
    lens = slot_lens or {}
    rows = range(batch)
    if any(not (0 <= slots[r] < n_slots) for r in rows):
        return SLOT
    if len(set(slots[r] for r in rows)) != batch:
        return INVALID
    if any(not (0 <= tokens[r] < cfg["vocab"]) for r in rows):
        return TOKEN
    if any(pos[r] < 0 or pos[r] + n_steps > cfg["max_seq"] for r in rows):
        return POSITION
    if any(pos[r] != lens.get(slots[r], 0) for r in rows):
        return CACHE_LEN
    if any(pos[r] + n_steps > capacity for r in rows):
        return CAPACITY
    if logits and len_logits != batch * cfg["vocab"]:
        return LOGITS_LEN
    if (len_tokens if len_tokens is not None else n_steps * batch) != n_steps * batch:
        return OUTPUT_LEN
    if hidden and len_hidden != batch * cfg["n_layer"] * cfg["d"]:
        return OUTPUT_LEN
    return INVALID if ws_short else OK


def prefill(cfg: dict, n=1, tensors_ok=True, lens_ok=True, pool_ok=True, pool_dims_bad=False, batch_weights_ok=True,
            n_slots=1, capacity=0, slot=0, slot_len=0, tokens=(0,), pos0=0, len_tokens=None, logits=False,
            len_logits=0, hidden=False, len_hidden=0, ws_short=False):
    """Expected status of llmk_prefill: the checks of llmk_decode_step_batch for one slot whose rows are the
    n prompt tokens at positions pos0 .. pos0 + n - 1, with the last position's logits and hidden states."""
    c = config_check(**cfg)
    if c != OK:
        return c
    if n < 1:
        return EMPTY
    if n > MAX_DIM:
        return TOO_LARGE
    if not tensors_ok:
        return INVALID
    if not lens_ok:
        return WEIGHT_LEN
    if not pool_ok:
        return INVALID
    if pool_dims_bad:
        return EMPTY
    if not batch_weights_ok:
        return INVALID
    if not (0 <= slot < n_slots):
        return SLOT
    if any(not (0 <= t < cfg["vocab"]) for t in tokens):
        return TOKEN
    if pos0 < 0 or pos0 + n > cfg["max_seq"]:
        return POSITION
    if pos0 != slot_len:
        return CACHE_LEN
    if pos0 + n > capacity:
        return CAPACITY
    if (len_tokens if len_tokens is not None else n) != n:
        return OUTPUT_LEN
    if logits and len_logits != cfg["vocab"]:
        return LOGITS_LEN
    if hidden and len_hidden != cfg["n_layer"] * cfg["d"]:
        return OUTPUT_LEN
    return INVALID if ws_short else OK
