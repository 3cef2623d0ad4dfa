"""Paged K/V pool on the GPU against the oracle's block manager and paged store (MI355X only).

"Inside the engine" (cajeta.dev), "3. The K/V cache and the block store": blocks of block_tokens positions,
shared by reference count after a fork and copied on the first write, refusal when the pool is full;
"2. The scheduler: continuous batching", "Admission".

1. Bookkeeping and copies: seeded random reserve / fork / release runs on a small pool. After every operation
   the library's table, reference counts and free count equal the oracle block manager's (the same rules,
   written independently), the device table equals the host mirror, and every live sequence reads back exactly
   the rows it was given (so copy-on-write copied the right block and nothing wrote into a shared one).
2. Decoding through the table: prefill, forks, single steps on the persistent and the per-operation form, a
   batched step whose rows copy and take blocks, captured multi-step runs crossing block boundaries, release,
   reuse, refusal when full (571, nothing changed) and admission. Every step's logits and hidden states are
   compared with the oracle's paged store fed the same tokens (within 2e-3, greedy tokens equal or a reported
   near-tie), the block tables with the oracle's, the cached K/V with the oracle's, and the logits of the
   single and batched steps bit for bit with the same calls on a contiguous pool.
"""
import random

import numpy as np
import pytest

import oracle
import synth
from oracle import contract
from oracle.paged import BlockManager, PagedStore
from tests.gpu_util import TOL, dev, host, rel_err, say, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402

BT = 64


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def same_state(pool, bm):
    assert pool.table_h.tolist() == bm.table
    assert pool.refcount.tolist() == bm.ref
    assert pool.n_free == bm.n_free()
    torch.cuda.synchronize()
    dt = host(pool.table).reshape(pool.n_slots, pool.max_blocks)
    held = pool.table_h >= 0
    assert np.array_equal(dt[held], pool.table_h[held]), "device table differs from the host mirror"


def test_block_manager_and_copies_match_oracle():
    rng = random.Random(17)
    n_slots, cap, n_blocks = 5, 5 * BT, 12
    pool = llmk.KVPool(2, n_slots, cap, 1, 4, llmk.F32, block_tokens=BT, n_blocks=n_blocks)
    bm = BlockManager(n_slots, cap, n_blocks, BT)
    hist = {s: np.zeros((0, 2, 2, 4), np.float32) for s in range(n_slots)}   # [pos][layer][k|v][4]
    next_val = [1.0]

    def rows(n):
        v = np.arange(next_val[0], next_val[0] + n * 16, dtype=np.float32).reshape(n, 2, 2, 4)
        next_val[0] += n * 16
        return v

    for op_i in range(160):
        s = rng.randrange(n_slots)
        r = rng.random()
        if r < 0.55:
            n = rng.choice([1, 1, 3, 40, 70])
            b = int(pool.slot_len[s])
            want, _ = bm.reserve([(s, b, b + n)])
            got = llmk.kv_reserve(pool, s, b, b + n)
            assert got == want, (op_i, s, b, n)
            if got == llmk.OK:
                v = rows(n)
                for l in range(2):
                    pool.write_positions(l, s, "k", b, torch.from_numpy(v[:, l, 0].reshape(n, 1, 4)).cuda())
                    pool.write_positions(l, s, "v", b, torch.from_numpy(v[:, l, 1].reshape(n, 1, 4)).cuda())
                pool.set_len(s, b + n)
                bm.length[s] = b + n
                hist[s] = np.concatenate([hist[s], v])
        elif r < 0.75:
            d = rng.randrange(n_slots)
            if d == s or pool.slot_len[s] == 0:
                continue
            if rng.random() < 0.6:
                assert llmk.kv_release(pool, d) == llmk.OK
                bm.release(d)
                hist[d] = hist[d][:0]
            n = rng.randint(1, int(pool.slot_len[s]))
            want = bm.fork(s, d, n)
            assert llmk.kv_fork(pool, s, d, n) == want
            if want == llmk.OK:
                hist[d] = hist[s][:n].copy()
        else:
            assert llmk.kv_release(pool, s) == llmk.OK
            bm.release(s)
            hist[s] = hist[s][:0]
        same_state(pool, bm)
        for q in range(n_slots):
            n = int(pool.slot_len[q])
            assert n == bm.length[q] == hist[q].shape[0]
            for l in range(2):
                k = host(pool.read_positions(l, q, "k", 0, n)).reshape(n, 4)
                v = host(pool.read_positions(l, q, "v", 0, n)).reshape(n, 4)
                assert np.array_equal(k, hist[q][:, l, 0]) and np.array_equal(v, hist[q][:, l, 1]), (op_i, q, l)
    say(f"block manager: 160 operations, {bm.n_free()} blocks free at the end")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_paged_pool_append_offsets_and_attend(dt):
    """llmk_kv_append and llmk_gqa_attend on a paged pool: appends of one position, of several positions across
    a block boundary and of part of a position; every returned offset equals the oracle's (its block manager's
    table), the values read back through the table are the oracle's rounding, a fork followed by an append
    copies the shared block and leaves the source's values alone, and attention over the slot equals the
    oracle's at several context lengths."""
    n_layer, n_slots, cap, Hkv, hd, H, n_blocks = 2, 3, 3 * BT, 2, 64, 8, 6
    kv = llmk.BF16 if dt == "bf16" else llmk.F32
    npdt = np.uint16 if dt == "bf16" else np.float32
    pool = llmk.KVPool(n_layer, n_slots, cap, Hkv, hd, kv, block_tokens=BT, n_blocks=n_blocks)
    bm = BlockManager(n_slots, cap, n_blocks, BT)
    row = Hkv * hd
    fields = dict(n_layer=n_layer, n_slots=n_slots, capacity=cap, n_kv=Hkv, head_dim=hd, dtype=kv,
                  pages=dict(block_tokens=BT, n_blocks=n_blocks, max_blocks=3))
    slot, layer = 2, 1
    n_el = 140 * row + 37                       # 140 whole positions and part of one more
    vals = {w: synth.normal((n_el,), 50 + w, 0, 1.0) for w in (0, 1)}
    chunks = [row] * 60 + [5 * row] + [row * 70, 5 * row + 37]    # 60, 65, 135, 140 positions and a part
    cl = 0
    for n_new in chunks:
        for w in (0, 1):
            p0, p_end = cl // row, -(-(cl + n_new) // row)
            if w == 0:
                before_free = bm.n_free()
                st_o, _ = bm.reserve([(slot, p0, p_end)])
                assert st_o == contract.OK
                need = before_free - bm.n_free()
            else:
                need = 0
            exp = contract.kv_append(fields, layer, slot, w, cl, cl, True, n_new, n_new, need=need,
                                     n_free=pool.n_free, row_of=lambda p: bm.row(slot, p))
            got = llmk.kv_append(pool, layer, slot, w, cl, dev(vals[w][cl:cl + n_new]))
            assert got == exp, (cl, n_new, w)
        cl += n_new
        same_state(pool, bm)
    _ = host(pool.k[0])
    for w, name in ((0, "k"), (1, "v")):
        got = host(pool.read_positions(layer, slot, name, 0, 141)).ravel()[:n_el]
        ref = oracle.kv_append_copy(np.zeros(0, npdt), vals[w], dt)
        assert np.array_equal(got, ref), name
    # attention over the slot against the oracle on the oracle's own K/V
    for ctx in (1, 33, 64, 65, 140):
        q = synth.normal((H * hd,), 51, ctx, 1.0)
        kk = oracle.kv_append_copy(np.zeros(0, npdt), vals[0][:ctx * row], dt)
        vv = oracle.kv_append_copy(np.zeros(0, npdt), vals[1][:ctx * row], dt)
        out = torch.full((H * hd,), float("nan"), dtype=torch.float32, device="cuda")
        ws = llmk.workspace(llmk.gqa_attend_workspace_bytes(ctx, H, hd))
        assert llmk.gqa_attend(dev(q), pool, layer, slot, ctx, H, out, ws) == llmk.OK
        torch.cuda.synchronize()
        ref = oracle.attend_f32(q, kk.reshape(ctx, Hkv, hd), vv.reshape(ctx, Hkv, hd), ctx, H, Hkv, hd)
        assert rel_err(host(out), ref) <= TOL, ctx
    # fork slot 2 into slot 0 at 100 positions, then an append to slot 0 copies the shared block 1
    pool.set_len(slot, 140)
    bm.length[slot] = 140
    assert llmk.kv_fork(pool, slot, 0, 100) == bm.fork(slot, 0, 100) == llmk.OK
    new0 = synth.normal((row,), 52, 0, 1.0)
    for l in range(n_layer):
        for w in (0, 1):
            if l == 0 and w == 0:
                st_o, copies = bm.reserve([(0, 100, 101)])
                assert st_o == contract.OK and len(copies) == 1
            exp = contract.kv_append(fields, l, 0, w, 100 * row, 100 * row, True, row, row,
                                     need=1 if (l, w) == (0, 0) else 0, n_free=pool.n_free,
                                     row_of=lambda p: bm.row(0, p))
            assert llmk.kv_append(pool, l, 0, w, 100 * row, dev(new0)) == exp, (l, w)
    same_state(pool, bm)
    for w, name in ((0, "k"), (1, "v")):
        src = host(pool.read_positions(layer, slot, name, 0, 141)).ravel()[:n_el]
        assert np.array_equal(src, oracle.kv_append_copy(np.zeros(0, npdt), vals[w], dt)), "source changed"
        fork = host(pool.read_positions(layer, 0, name, 0, 101)).ravel()
        ref = oracle.kv_append_copy(np.zeros(0, npdt), np.concatenate([vals[w][:100 * row], new0]), dt)
        assert np.array_equal(fork, ref), "forked slot"


# ---- decoding through the table ------------------------------------------------------------------------

PAGED = synth.Shape("paged test decoder bf16 (V512 d256 L2 H4/2 hd128 F512)", 512, 256, 2, 4, 2, 128, 512, 512,
                    1e-5, 1e4, synth.ROPE_HALF_SPLIT, "bf16", "bf16", 0.05)


def near_tie(logits, tol=TOL):
    s = np.sort(np.asarray(logits, np.float64))
    return (s[-1] - s[-2]) <= 2 * tol * np.max(np.abs(s))


class Oracle:
    """The oracle's paged store over the same operations, fed the GPU's tokens."""

    def __init__(self, s, W, n_slots, n_blocks):
        self.m = oracle.Model(s, W)
        self.st = PagedStore(s, n_slots, s.max_seq, n_blocks, BT)
        self.scratch = self.m.new_cache(s.max_seq)
        self.ties = []

    def step(self, slot, token, g_logits=None, g_hidden=None, g_next=None, label=""):
        st, lg, hd = self.st.step(self.m, slot, int(token), self.scratch, want_hidden=True)
        assert st == oracle.paged.OK
        if g_logits is not None:
            el, eh = rel_err(g_logits, lg), rel_err(g_hidden, hd)
            assert el <= TOL and eh <= TOL, f"{label}: logits {el:.2e} hidden {eh:.2e}"
        if g_next is not None and int(g_next) != oracle.argmax(lg)[0]:
            assert near_tie(lg), f"{label}: token {g_next} != oracle {oracle.argmax(lg)[0]}"
            self.ties.append(label)
        return lg


def kv_close(got, ref):
    g, w = oracle.widen(got), oracle.widen(ref)
    mag = np.where(w != 0, np.abs(w), 1e-38)
    bar = np.maximum(TOL * np.max(np.abs(w)), np.exp2(np.floor(np.log2(mag)) - 7))
    return not (np.abs(g - w) > bar).any()


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_paged_decoding_matches_oracle_and_contiguous(kv):
    s = PAGED.with_(kv_dtype=kv)
    W = weights(s, seed=9)
    n_slots, n_blocks = 4, 8
    cfg = loader.config_from(s)
    cfg_op = loader.config_from(s, step_path=llmk.STEP_PER_OP)
    assert llmk.decode_path(cfg) == llmk.STEP_PERSISTENT
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, n_slots, s.max_seq, block_tokens=BT, n_blocks=n_blocks)
    flat = loader.new_pool(cfg, n_slots, s.max_seq)          # the same calls on a contiguous pool
    O = Oracle(s, W, n_slots, n_blocks)
    A, B, C, D = 0, 1, 2, 3
    prompt = synth.prompt(100, s.vocab, stream=41).tolist()
    V, Ld = s.vocab, s.n_layer * s.d

    def bufs(rows=1):
        return (torch.full((rows * V,), float("nan"), device="cuda"), torch.full((rows * Ld,), float("nan"), device="cuda"))

    say(f"[{kv}] prefill A (100 tokens) on both pools")
    outs = []
    for p in (pool, flat):
        tok = torch.full((100,), -1, dtype=torch.int32, device="cuda")
        lg, hd = bufs()
        ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, 100))
        assert llmk.prefill(cfg, model, p, A, prompt, 0, tok, ws, lg, hd) == llmk.OK
        torch.cuda.synchronize()
        outs.append((host(tok).tolist(), host(lg), host(hd)))
    assert outs[0][0] == outs[1][0] and np.array_equal(outs[0][1], outs[1][1]), "paged prefill != contiguous"
    for i, t in enumerate(prompt):
        lg = O.step(A, t, *((outs[0][1], outs[0][2].reshape(s.n_layer, s.d)) if i == 99 else (None, None)),
                    g_next=outs[0][0][i], label=f"prefill {i}")
    same_state(pool, O.st.bm)
    a_next = outs[0][0][-1]

    say(f"[{kv}] fork B from A at 100 (block 1 shared half full), one step each: persistent A, per-operation B")
    assert llmk.kv_fork(pool, A, B, 100) == O.st.bm.fork(A, B, 100) == llmk.OK
    for l in range(s.n_layer):                                 # the contiguous pool copies the prefix
        for w in ("k", "v"):
            flat.slot_view(l, B, w)[:100] = flat.slot_view(l, A, w)[:100]
    flat.set_len(B, 100)
    b_first = int(synth.prompt(1, s.vocab, stream=42)[0])
    dec = {p: loader.Decoder(cfg, model, p) for p in (pool, flat)}
    dec_op = {p: loader.Decoder(cfg_op, model, p) for p in (pool, flat)}
    res = {}
    for p in (pool, flat):
        lg_a, hd_a = bufs()
        assert dec[p].step(a_next, 100, A, lg_a, hd_a) == llmk.OK
        torch.cuda.synchronize()
        ta = int(host(dec[p].token_out)[0])
        lg_b, hd_b = bufs()
        assert dec_op[p].step(b_first, 100, B, lg_b, hd_b) == llmk.OK
        torch.cuda.synchronize()
        tb = int(host(dec_op[p].token_out)[0])
        res[p] = (ta, host(lg_a), host(hd_a), tb, host(lg_b), host(hd_b))
    for i in (0, 1, 3, 4):
        assert np.array_equal(res[pool][i], res[flat][i]), f"single step output {i}: paged != contiguous"
    ta, lga, hda, tb, lgb, hdb = res[pool]
    O.step(A, a_next, lga, hda.reshape(s.n_layer, s.d), ta, "A step 100")
    O.step(B, b_first, lgb, hdb.reshape(s.n_layer, s.d), tb, "B step 100")
    same_state(pool, O.st.bm)
    assert pool.table_h[A, 1] != pool.table_h[B, 1], "A's write did not copy the shared block"

    say(f"[{kv}] fork C from A at 50, batched step A, B, C (C copies block 0)")
    assert llmk.kv_fork(pool, A, C, 50) == O.st.bm.fork(A, C, 50) == llmk.OK
    for l in range(s.n_layer):
        for w in ("k", "v"):
            flat.slot_view(l, C, w)[:50] = flat.slot_view(l, A, w)[:50]
    flat.set_len(C, 50)
    c_first = int(synth.prompt(1, s.vocab, stream=43)[0])
    slots, toks, poss = [A, B, C], [ta, tb, c_first], [101, 101, 50]
    bres = {}
    for p in (pool, flat):
        bd = loader.BatchDecoder(cfg, model, p, 3)
        lg, hd = bufs(3)
        assert bd.step(slots, toks, poss, lg, hd) == llmk.OK
        torch.cuda.synchronize()
        bres[p] = (host(bd.tokens_out).tolist(), host(lg).reshape(3, V), host(hd).reshape(3, s.n_layer, s.d))
    assert bres[pool][0] == bres[flat][0] and np.array_equal(bres[pool][1], bres[flat][1]), "batched: paged != flat"
    for r in range(3):
        O.step(slots[r], toks[r], bres[pool][1][r], bres[pool][2][r], bres[pool][0][r], f"batched row {r}")
    same_state(pool, O.st.bm)

    say(f"[{kv}] captured runs: A 40 steps from 102 (crosses 128), B and C 20 batched steps (C crosses 64)")
    out = torch.zeros(40, dtype=torch.int32, device="cuda")
    assert dec[pool].steps(bres[pool][0][0], 102, 40, out, slot=A) == llmk.OK
    torch.cuda.synchronize()
    a_toks = host(out).tolist()
    fed = [bres[pool][0][0]] + a_toks[:-1]
    for i, t in enumerate(fed):
        O.step(A, t, g_next=a_toks[i], label=f"A graph step {i}")
    bd = loader.BatchDecoder(cfg, model, pool, 2)
    out2 = torch.zeros(40, dtype=torch.int32, device="cuda")
    assert bd.steps([B, C], bres[pool][0][1:], [102, 51], 20, out2) == llmk.OK
    torch.cuda.synchronize()
    bc = host(out2).reshape(20, 2)
    for j in range(20):
        for r, sl in enumerate((B, C)):
            t = bres[pool][0][1 + r] if j == 0 else int(bc[j - 1, r])
            O.step(sl, t, g_next=int(bc[j, r]), label=f"batched graph step {j} row {r}")
    same_state(pool, O.st.bm)
    say(f"[{kv}] tables {pool.table_h.tolist()}, refcounts {pool.refcount.tolist()}")

    # the cached K/V of every live sequence, read through the table, against the oracle's store
    for sl in (A, B, C):
        n = int(pool.slot_len[sl])
        O.st.gather(sl, n, O.scratch)
        for l in range(s.n_layer):
            for w, ref in (("k", O.scratch.k[l]), ("v", O.scratch.v[l])):
                assert kv_close(host(pool.read_positions(l, sl, w, 0, n)), ref[:n]), (sl, l, w)

    say(f"[{kv}] release B, prefill D (reuses B's freed block), refusal when full, admission")
    assert llmk.kv_release(pool, B) == llmk.OK
    O.st.bm.release(B)
    d_prompt = synth.prompt(30, s.vocab, stream=44).tolist()
    tok = torch.full((30,), -1, dtype=torch.int32, device="cuda")
    lg, hd = bufs()
    ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, 30))
    assert llmk.prefill(cfg, model, pool, D, d_prompt, 0, tok, ws, lg, hd) == llmk.OK
    torch.cuda.synchronize()
    d_toks = host(tok).tolist()
    for i, t in enumerate(d_prompt):
        O.step(D, t, *((host(lg), host(hd).reshape(s.n_layer, s.d)) if i == 29 else (None, None)),
               g_next=d_toks[i], label=f"D prefill {i}")
    same_state(pool, O.st.bm)
    free = pool.n_free
    st_o, _ = O.st.bm.reserve([(D, 30, 30 + BT * (free + 1))])
    assert llmk.kv_reserve(pool, D, 30, 30 + BT * (free + 1)) == st_o == llmk.CACHE_CAPACITY_EXCEEDED
    same_state(pool, O.st.bm)
    assert llmk.kv_reserve(pool, D, 30, 30 + BT * free) == llmk.OK   # takes the rest
    O.st.reserve([(D, 30, 30 + BT * free)])
    assert pool.n_free == 0
    assert llmk.kv_admit(pool, 0) == (llmk.OK, 0)
    # B forks A again; its first step needs a copy of A's shared last block and none is free
    n_a = int(pool.slot_len[A])
    assert llmk.kv_fork(pool, A, B, n_a) == O.st.bm.fork(A, B, n_a) == llmk.OK
    before = (pool.table_h.copy(), pool.refcount.copy(), int(pool.slot_len[B]))
    lg, hd = bufs()
    assert dec[pool].step(0, n_a, B, lg, hd) == llmk.CACHE_CAPACITY_EXCEEDED
    assert np.array_equal(before[0], pool.table_h) and np.array_equal(before[1], pool.refcount)
    assert int(pool.slot_len[B]) == before[2]
    same_state(pool, O.st.bm)
    assert llmk.kv_release(pool, D) == llmk.OK
    O.st.bm.release(D)
    nf = pool.n_free
    assert llmk.kv_admit(pool, BT * (nf - 1)) == (llmk.OK, 1) and llmk.kv_admit(pool, BT * (nf - 1) + 1) == (llmk.OK, 0)
    same_state(pool, O.st.bm)
    say(f"[{kv}] near-ties (reported): {O.ties}")
