"""The batched decode step (several sequences per step, matrix-core projections) against the oracle.

Every row of a batch is an independent sequence: its own slot, context length, token and position. The
oracle runs each row on its own cache; the GPU runs all rows in one call. Per row: greedy token bit-exact
(or a reported near-tie), logits and per-layer hidden states within the bar, the K/V it appends at the
closed-form offsets of its slot, and no other pool position changed. Multi-step calls must reproduce the
oracle's free-running tokens.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, host, rel_err, say, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def near_tie(logits, tol=TOL):
    s = np.sort(np.asarray(logits, np.float64))
    return (s[-1] - s[-2]) <= 2 * tol * np.max(np.abs(s))


TINY_BF16 = synth.TINY.with_(name="tiny-llama bf16 weights", w_dtype="bf16")


def setup(shape, W, n_slots, capacity):
    cfg = loader.config_from(shape)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, n_slots, capacity)
    return cfg, model, pool


def check_rows(shape, m, caches, rows, slots, tokens, pos, g_logits, g_hidden, g_tokens, label):
    """Oracle step for each listed row on its own cache; compare with the GPU's outputs of that row."""
    worst = 0.0
    for r in rows:
        lg, hid = m.forward_token(int(tokens[r]), int(pos[r]), caches[r], want_hidden=True)
        el = rel_err(g_logits[r], lg)
        eh = rel_err(g_hidden[r], hid)
        worst = max(worst, el, eh)
        assert el <= TOL, f"{label} row {r}: logits rel err {el:.3e}"
        assert eh <= TOL, f"{label} row {r}: hidden rel err {eh:.3e}"
        want = oracle.argmax(lg)[0]
        if int(g_tokens[r]) != want:
            assert near_tie(lg), f"{label} row {r}: token {int(g_tokens[r])} != oracle {want}"
            say(f"{label} row {r}: near-tie, gpu {int(g_tokens[r])} oracle {want}")
    say(f"{label}: {len(rows)} rows, worst rel err {worst:.2e}")


def test_tiny_batch_matches_oracle_per_row():
    s = TINY_BF16
    W = weights(s)
    ctxs = [0, 3, 17, 40, 9]
    slots = [4, 0, 2, 1, 3]
    B = len(slots)
    cfg, model, pool = setup(s, W, n_slots=6, capacity=s.max_seq)
    m = oracle.Model(s, W)
    caches = []
    for r in range(B):
        pre = synth.kv_prefix(s, max(ctxs[r], 1), seed=2, slot=r)
        if ctxs[r] > 0:
            pre = [(k[:ctxs[r]], v[:ctxs[r]]) for k, v in pre]
            loader.fill_prefix(pool, slots[r], pre)
        c = m.new_cache(s.max_seq)
        if ctxs[r] > 0:
            c.fill_prefix(pre)
        caches.append(c)
    before = {l: (host(pool.k[l]).copy(), host(pool.v[l]).copy()) for l in range(s.n_layer)}
    tokens = synth.prompt(B, s.vocab, stream=11).tolist()
    dec = loader.BatchDecoder(cfg, model, pool, B)
    lg = torch.full((B * s.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    hd = torch.full((B * s.n_layer * s.d,), float("nan"), dtype=torch.float32, device="cuda")
    assert dec.step(slots, tokens, ctxs, lg, hd) == llmk.OK
    torch.cuda.synchronize()
    g_tok = host(dec.tokens_out).tolist()
    check_rows(s, m, caches, range(B), slots, tokens, ctxs, host(lg).reshape(B, -1),
               host(hd).reshape(B, s.n_layer, s.d), g_tok, "tiny batch")
    assert [int(pool.slot_len[slots[r]]) for r in range(B)] == [c + 1 for c in ctxs]
    # the appended K/V of each row sits at its slot's closed-form offset for its position (values within
    # the bar of the oracle's); every other element of the pool is unchanged, bit for bit
    for l in range(s.n_layer):
        for which, now, was in (("k", host(pool.k[l]), before[l][0]), ("v", host(pool.v[l]), before[l][1])):
            changed = np.zeros(now.shape[0], bool)
            for r in range(B):
                for kvh in range(s.n_kv):
                    st, off = llmk.kv_slot_offset(pool, slots[r], ctxs[r], kvh)
                    assert st == llmk.OK
                    exp_st, exp_off = oracle.contract.kv_slot_offset(6, s.max_seq, s.n_kv, s.head_dim, slots[r],
                                                                     ctxs[r], kvh)
                    assert off == exp_off
                    ref = (caches[r].k if which == "k" else caches[r].v)[l][ctxs[r], kvh]
                    assert rel_err(kv_vals(now[off:off + s.head_dim]), kv_vals(ref)) <= TOL
                    changed[off:off + s.head_dim] = True
            assert np.array_equal(now[~changed], was[~changed])

    # free-running: 6 more steps of every row in one call against the oracle's greedy continuation
    n = 6
    out = torch.zeros(n * B, dtype=torch.int32, device="cuda")
    pos1 = [c + 1 for c in ctxs]
    assert dec.steps(slots, g_tok, pos1, n, out) == llmk.OK
    got = host(out).reshape(n, B)
    for r in range(B):
        t, want = g_tok[r], []
        for i in range(n):
            lgo, _ = m.forward_token(t, pos1[r] + i, caches[r])
            t = oracle.argmax(lgo)[0]
            want.append(t)
        assert got[:, r].tolist() == want, f"row {r}"


def kv_vals(a):
    """K/V values as float64 (bf16 pools hold uint16 bit patterns)."""
    a = np.asarray(a)
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def test_batch_of_one_equals_single_sequence_step():
    s = TINY_BF16
    W = weights(s)
    cfg, model, pool = setup(s, W, n_slots=2, capacity=s.max_seq)
    pre = synth.kv_prefix(s, 11, seed=2)
    for slot in (0, 1):
        loader.fill_prefix(pool, slot, pre)
    single = loader.Decoder(cfg, model, pool)
    batch = loader.BatchDecoder(cfg, model, pool, 1)
    toks_a, toks_b = [5], [5]
    for i in range(8):
        assert single.step(toks_a[-1], 11 + i, 0) == llmk.OK
        assert batch.step([1], [toks_b[-1]], [11 + i]) == llmk.OK
        torch.cuda.synchronize()
        toks_a.append(int(host(single.token_out)[0]))
        toks_b.append(int(host(batch.tokens_out)[0]))
    assert toks_a == toks_b


@pytest.fixture(scope="module")
def q06():
    s = synth.Q06
    say("generating Qwen3-0.6B-shaped weights")
    return s, weights(s)


def test_q06_batch_of_16_ragged(q06):
    s, W = q06
    B = 16
    ctxs = synth.ragged_contexts(B, 0, 300, seed=3).tolist()
    slots = list(range(B))[::-1]
    cap = 320
    cfg, model, pool = setup(s, W, n_slots=B, capacity=cap)
    m = oracle.Model(s, W)
    src = synth.kv_prefix(s, max(ctxs) + synth.slot_window(B), seed=2)
    src_dev = loader.upload_kv_source(src)
    caches = []
    for r in range(B):
        st = synth.slot_window(r)
        loader.fill_prefix_window(pool, slots[r], src_dev, st, ctxs[r])
        c = m.new_cache(cap)
        if ctxs[r] > 0:
            c.fill_prefix([(k[st:st + ctxs[r]], v[st:st + ctxs[r]]) for k, v in src])
        caches.append(c)
    tokens = synth.prompt(B, s.vocab, stream=12).tolist()
    dec = loader.BatchDecoder(cfg, model, pool, B)
    lg = torch.empty(B * s.vocab, dtype=torch.float32, device="cuda")
    hd = torch.empty(B * s.n_layer * s.d, dtype=torch.float32, device="cuda")
    assert dec.step(slots, tokens, ctxs, lg, hd) == llmk.OK
    torch.cuda.synchronize()
    g_tok = host(dec.tokens_out).tolist()
    check_rows(s, m, caches, range(B), slots, tokens, ctxs, host(lg).reshape(B, -1),
               host(hd).reshape(B, s.n_layer, s.d), g_tok, "q06 batch 16")
    n = 3
    out = torch.zeros(n * B, dtype=torch.int32, device="cuda")
    pos1 = [c + 1 for c in ctxs]
    assert dec.steps(slots, g_tok, pos1, n, out) == llmk.OK
    got = host(out).reshape(n, B)
    for r in range(B):
        t, want = g_tok[r], []
        for i in range(n):
            lgo, _ = m.forward_token(t, pos1[r] + i, caches[r])
            t = oracle.argmax(lgo)[0]
            want.append(t)
        assert got[:, r].tolist() == want, f"row {r}"
