"""Pins of the oracle's paged K/V cache (oracle/paged.py) against what the page fixes, on the CPU.

"Inside the engine" (cajeta.dev), "3. The K/V cache and the block store" (fixed blocks, shared by reference
count with copy-on-write, refusal when full) and "2. The scheduler: continuous batching", "Admission".

  - a worked example, derived by hand from those rules, with every table, reference count and copy spelled out;
  - invariants after every operation of seeded random runs (a block's count equals the table entries that hold
    it, the free count equals the blocks nobody holds, no slot holds a block twice, a refusal changes nothing);
  - content: a paged store driven by random appends and forks holds, for every live sequence, exactly the rows
    a plain per-sequence list received (a missing copy, a copy of the wrong block or a table off by one fails);
  - the oracle's decode step taken through the paged store gives bit-identical logits and hidden states to
    independent contiguous caches, for two sequences forked from a common prefix (the paged layout changes
    nothing the step computes).
"""
import copy
import random

import numpy as np

import oracle
import synth
from oracle.paged import CACHE_LENGTH_MISMATCH, CAPACITY_EXCEEDED, OK, BlockManager, PagedStore


def state(bm):
    return copy.deepcopy((bm.table, bm.ref, bm.length))


def check_invariants(bm):
    held = [0] * bm.n_blocks
    for row in bm.table:
        live = [b for b in row if b != -1]
        assert len(live) == len(set(live)), "a slot holds a block twice"
        for b in live:
            assert 0 <= b < bm.n_blocks
            held[b] += 1
    assert held == bm.ref
    assert bm.n_free() == sum(1 for h in held if h == 0)


def test_worked_example():
    bm = BlockManager(n_slots=3, capacity=16, n_blocks=6, block_tokens=4)
    A, B, C = 0, 1, 2
    assert bm.reserve([(A, 0, 6)]) == (OK, [])
    bm.length[A] = 6
    assert bm.table[A] == [0, 1, -1, -1] and bm.ref == [1, 1, 0, 0, 0, 0]
    assert bm.fork(A, B, 6) == OK
    assert bm.table[B] == [0, 1, -1, -1] and bm.ref == [2, 2, 0, 0, 0, 0] and bm.length[B] == 6
    # A writes position 6 into the shared block 1: its own copy in block 2
    assert bm.reserve([(A, 6, 7)]) == (OK, [(1, 2)])
    bm.length[A] = 7
    assert bm.table[A] == [0, 2, -1, -1] and bm.ref == [2, 1, 1, 0, 0, 0]
    # B is now block 1's only holder: written in place, then a fresh block for positions 8..
    assert bm.reserve([(B, 6, 7)]) == (OK, [])
    assert bm.reserve([(B, 7, 9)]) == (OK, [])
    bm.length[B] = 9
    assert bm.table[B] == [0, 1, 3, -1] and bm.ref == [2, 1, 1, 1, 0, 0]
    assert bm.fork(A, C, 7) == OK
    assert bm.table[C] == [0, 2, -1, -1] and bm.ref == [3, 1, 2, 1, 0, 0]
    # C needs a copy of block 2 and two fresh blocks; two are free: refused, nothing changed
    before = state(bm)
    assert bm.reserve([(C, 7, 13)]) == (CAPACITY_EXCEEDED, [])
    assert state(bm) == before
    assert bm.reserve([(C, 7, 12)]) == (OK, [(2, 4)])
    assert bm.table[C] == [0, 4, 5, -1] and bm.ref == [3, 1, 1, 1, 1, 1] and bm.n_free() == 0
    # admission: an empty suffix still needs its block of headroom
    assert not bm.admit(0)
    bm.release(A)
    assert bm.table[A] == [-1] * 4 and bm.ref == [2, 1, 0, 1, 1, 1] and bm.length[A] == 0
    assert bm.admit(0) and not bm.admit(1)
    # fork refusals: dst not empty, more positions than src holds
    assert bm.fork(B, C, 3) == CACHE_LENGTH_MISMATCH
    assert bm.fork(B, A, 10) == CACHE_LENGTH_MISMATCH
    bm.release(B)
    bm.release(C)
    assert bm.ref == [0] * 6 and bm.n_free() == 6
    assert bm.admit(20) and not bm.admit(21)          # ceil(20 / 4) + 1 = 6, ceil(21 / 4) + 1 = 7
    # past the capacity: refused whatever is free
    assert bm.reserve([(A, 0, 17)]) == (CAPACITY_EXCEEDED, [])


def test_two_requests_one_call_share_the_count():
    # rows of one batched call: the first copy leaves the second writer the only holder, which writes in place
    bm = BlockManager(n_slots=2, capacity=8, n_blocks=3, block_tokens=4)
    bm.reserve([(0, 0, 3)])
    bm.length[0] = 3
    bm.fork(0, 1, 3)
    assert bm.reserve([(0, 3, 4), (1, 3, 4)]) == (OK, [(0, 1)])
    assert bm.table[0][:1] == [1] and bm.table[1][:1] == [0] and bm.ref == [1, 1, 0]


def test_random_runs_keep_the_invariants():
    rng = random.Random(11)
    for run in range(40):
        bt = rng.choice([1, 2, 4])
        bm = BlockManager(n_slots=5, capacity=24, n_blocks=rng.randint(3, 14), block_tokens=bt)
        for _ in range(60):
            op = rng.random()
            s = rng.randrange(5)
            if op < 0.55:
                n = rng.randint(1, 6)
                before = state(bm)
                st, _ = bm.reserve([(s, bm.length[s], bm.length[s] + n)])
                if st == OK:
                    bm.length[s] += n
                else:
                    assert st == CAPACITY_EXCEEDED and state(bm) == before
            elif op < 0.75:
                d = rng.randrange(5)
                if d != s and bm.length[s] > 0:
                    before = state(bm)
                    st = bm.fork(s, d, rng.randint(1, bm.length[s]))
                    if st != OK:
                        assert state(bm) == before
            elif op < 0.9:
                bm.release(s)
            else:
                st, _ = bm.reserve([(x, bm.length[x], bm.length[x] + 1) for x in rng.sample(range(5), 3)])
            check_invariants(bm)


class _Tiny:
    n_layer, n_kv, head_dim, kv_dtype = 2, 1, 2, "f32"


def test_paged_store_holds_what_each_sequence_received():
    rng = random.Random(5)
    for run in range(25):
        st_ = PagedStore(_Tiny, n_slots=4, capacity=20, n_blocks=rng.randint(6, 16), block_tokens=rng.choice([2, 4]))
        plain = {s: [] for s in range(4)}       # each sequence's rows, as appended
        val = 0.0
        for _ in range(50):
            s = rng.randrange(4)
            if rng.random() < 0.7:
                pos = st_.bm.length[s]
                if st_.reserve([(s, pos, pos + 1)]) != OK:
                    continue
                rows = [(np.full((1, 2), val + 10 * l), np.full((1, 2), -val - 10 * l)) for l in range(2)]
                val += 1.0
                st_.write(s, pos, rows)
                st_.bm.length[s] = pos + 1
                plain[s].append(rows)
            else:
                d = rng.randrange(4)
                if d == s or st_.bm.length[s] == 0:
                    continue
                if rng.random() < 0.5:
                    st_.bm.release(d)
                    plain[d] = []
                n = rng.randint(1, st_.bm.length[s])
                if st_.bm.fork(s, d, n) == OK:
                    plain[d] = list(plain[s][:n])
            for q in range(4):
                for p, rows in enumerate(plain[q]):
                    r = st_.bm.row(q, p)
                    for l in range(2):
                        assert np.array_equal(st_.k[l][r], rows[l][0]) and np.array_equal(st_.v[l][r], rows[l][1])


def test_decode_through_paged_blocks_equals_contiguous_runs():
    s = synth.TINY
    W = synth.model(s, seed=4)
    m = oracle.Model(s, W)
    prompt = synth.prompt(7, s.vocab, stream=31).tolist()
    tail_a = synth.prompt(6, s.vocab, stream=32).tolist()
    tail_b = synth.prompt(6, s.vocab, stream=33).tolist()
    store = PagedStore(s, n_slots=2, capacity=16, n_blocks=9, block_tokens=4)
    scratch = m.new_cache(16)
    A, B = 0, 1
    for t in prompt:
        assert store.step(m, A, t, scratch)[0] == OK
    assert store.bm.fork(A, B, len(prompt)) == OK       # position 7 sits in the shared block 1
    got = {A: [], B: []}
    for i in range(6):                                  # interleaved, so each side writes into shared blocks
        for seq, tail in ((B, tail_b), (A, tail_a)):
            st, lg, hd = store.step(m, seq, tail[i], scratch, want_hidden=True)
            assert st == OK
            got[seq].append((lg, hd))
    check_invariants(store.bm)
    for seq, tail in ((A, tail_a), (B, tail_b)):
        c = m.new_cache(16)
        for p, t in enumerate(prompt):
            m.forward_token(t, p, c)
        for i, t in enumerate(tail):
            lg, hd = m.forward_token(t, len(prompt) + i, c, want_hidden=True)
            assert np.array_equal(lg, got[seq][i][0]) and np.array_equal(hd, got[seq][i][1]), (seq, i)
