"""THE ORACLE'S paged K/V cache -- test infrastructure only (tests/ may import it; the GPU library never does).

"Inside the engine" (cajeta.dev), "3. The K/V cache and the block store": the cache is cut into fixed blocks
of block_tokens positions; sequences that fork from a common prefix share its blocks, each block counting the
sequences that hold it, and a shared block is copied before one of them writes into it (copy-on-write); when
the pool has no block left the append refuses. "2. The scheduler: continuous batching", "Admission": a request
is admitted when the free blocks cover its whole uncached suffix plus one block of decode headroom for every
layer that is not windowed.

Readings where the page is silent (each also stated where the library documents its pool):
  - a block holds block_tokens positions of every layer's K and V, so the headroom is one block;
  - a request takes the lowest-numbered free block, requests are served in the order given and, within one,
    in block order;
  - a copy takes the whole block (every position, every layer, K and V);
  - a call that cannot get every block it needs changes nothing and reports the refusal (571).

BlockManager is the bookkeeping alone (tables, reference counts); PagedStore adds the cached values, one
array per (layer, K or V) of shape [n_blocks][block_tokens][n_kv][head_dim], and runs the oracle's decode
step of one sequence through its blocks: gather the sequence's positions into a contiguous cache, take the
step, scatter the new position back. Both are plain Python loops and numpy copies.
"""
from __future__ import annotations

import numpy as np

OK = 560
CACHE_LENGTH_MISMATCH = 566
CAPACITY_EXCEEDED = 571


class BlockManager:
    """Block tables of n_slots sequences over n_blocks blocks of block_tokens positions."""

    def __init__(self, n_slots: int, capacity: int, n_blocks: int, block_tokens: int):
        self.n_slots, self.capacity, self.n_blocks, self.bt = n_slots, capacity, n_blocks, block_tokens
        self.max_blocks = -(-capacity // block_tokens)
        self.table = [[-1] * self.max_blocks for _ in range(n_slots)]
        self.ref = [0] * n_blocks
        self.length = [0] * n_slots

    def n_free(self) -> int:
        return sum(1 for r in self.ref if r == 0)

    def _lowest_free(self) -> int:
        for b, r in enumerate(self.ref):
            if r == 0:
                return b
        raise AssertionError("no free block (the count was checked first)")

    def reserve(self, requests):
        """Make positions [begin, end) of each (slot, begin, end) writable. Returns (status, copies), copies the
        (from, to) block pairs to duplicate, in order; on a refusal nothing changes."""
        if any(end > self.capacity for _, _, end in requests):
            return CAPACITY_EXCEEDED, []
        # what the requests would take, walked on a copy of the state
        table = [list(row) for row in self.table]
        ref = list(self.ref)
        taken = 0
        for slot, begin, end in requests:
            for j in range(begin // self.bt, (end - 1) // self.bt + 1) if end > begin else ():
                b = table[slot][j]
                if b == -2:
                    continue
                if b == -1 or ref[b] > 1:
                    taken += 1
                    if b != -1:
                        ref[b] -= 1
                    table[slot][j] = -2          # marks the entry as owned for the rest of the walk
        if taken > self.n_free():
            return CAPACITY_EXCEEDED, []
        copies = []
        for slot, begin, end in requests:
            for j in range(begin // self.bt, (end - 1) // self.bt + 1) if end > begin else ():
                b = self.table[slot][j]
                if b != -1 and self.ref[b] == 1:
                    continue                     # private already: written in place
                nb = self._lowest_free()
                self.ref[nb] = 1
                if b != -1:                      # shared: the writer gets its own copy
                    self.ref[b] -= 1
                    copies.append((b, nb))
                self.table[slot][j] = nb
        return OK, copies

    def fork(self, src: int, dst: int, n_pos: int) -> int:
        """dst shares the blocks of src's first n_pos positions."""
        if n_pos > self.length[src] or self.length[dst] != 0 or any(b != -1 for b in self.table[dst]):
            return CACHE_LENGTH_MISMATCH
        for j in range(-(-n_pos // self.bt)):
            b = self.table[src][j]
            self.table[dst][j] = b
            self.ref[b] += 1
        self.length[dst] = n_pos
        return OK

    def release(self, slot: int) -> None:
        for j, b in enumerate(self.table[slot]):
            if b != -1:
                self.ref[b] -= 1
            self.table[slot][j] = -1
        self.length[slot] = 0

    def admit(self, n_uncached: int) -> bool:
        return self.n_free() >= -(-n_uncached // self.bt) + 1

    def row(self, slot: int, pos: int) -> int:
        """Cache row of a position (block * block_tokens + offset), -1 when its block is not reserved."""
        b = self.table[slot][pos // self.bt]
        return -1 if b == -1 else b * self.bt + pos % self.bt


class PagedStore:
    """The cached K/V of a BlockManager's sequences, per layer, in the shape's K/V dtype."""

    def __init__(self, shape, n_slots: int, capacity: int, n_blocks: int, block_tokens: int):
        self.shape = shape
        self.bm = BlockManager(n_slots, capacity, n_blocks, block_tokens)
        npdt = {"f32": np.float32, "bf16": np.uint16}[shape.kv_dtype]
        dims = (n_blocks * block_tokens, shape.n_kv, shape.head_dim)
        self.k = [np.zeros(dims, dtype=npdt) for _ in range(shape.n_layer)]
        self.v = [np.zeros(dims, dtype=npdt) for _ in range(shape.n_layer)]

    def reserve(self, requests) -> int:
        st, copies = self.bm.reserve(requests)
        bt = self.bm.bt
        for a, b in copies:
            for arr in self.k + self.v:
                arr[b * bt:(b + 1) * bt] = arr[a * bt:(a + 1) * bt]
        return st

    def write(self, slot: int, pos: int, layer_kv) -> None:
        """Store per layer (k, v) rows [n_kv][hd] at a reserved position."""
        r = self.bm.row(slot, pos)
        assert r >= 0, "position not reserved"
        for l, (kk, vv) in enumerate(layer_kv):
            self.k[l][r] = kk
            self.v[l][r] = vv

    def gather(self, slot: int, n: int, cache) -> None:
        """Positions 0..n-1 of a sequence into an oracle Cache (contiguous, the same dtype)."""
        for p in range(n):
            r = self.bm.row(slot, p)
            for l in range(self.shape.n_layer):
                cache.k[l][p] = self.k[l][r]
                cache.v[l][p] = self.v[l][r]
        cache.length = n

    def fill(self, slot: int, prefix) -> int:
        """Reserve and store a seeded prefix (per layer (K, V), each [n][n_kv][hd]) as positions 0..n-1."""
        n = prefix[0][0].shape[0]
        st = self.reserve([(slot, 0, n)])
        if st != OK:
            return st
        for p in range(n):
            self.write(slot, p, [(kk[p], vv[p]) for kk, vv in prefix])
        self.bm.length[slot] = n
        return OK

    def step(self, model, slot: int, token: int, scratch, want_hidden=False):
        """The oracle's decode step of one sequence through its blocks: the position it writes is reserved
        (a fresh or copied block), the sequence is gathered into `scratch` (an oracle Cache of at least pos + 1
        positions), the step runs there and its new K/V row is stored back. Returns (status, logits, hidden)."""
        pos = self.bm.length[slot]
        st = self.reserve([(slot, pos, pos + 1)])
        if st != OK:
            return st, None, None
        self.gather(slot, pos, scratch)
        logits, hidden = model.forward_token(token, pos, scratch, want_hidden)
        self.write(slot, pos, [(scratch.k[l][pos], scratch.v[l][pos]) for l in range(self.shape.n_layer)])
        self.bm.length[slot] = pos + 1
        return OK, logits, hidden
