"""Prefill (llmk_prefill) against the oracle and against the decode path (GPU).

A prompt chunk is a batch of rows of one slot at consecutive positions; the oracle defines the result as
the same tokens fed one decode step at a time. Checked: the greedy token after every position (bit-exact,
or a reported near-tie), the last position's logits and per-layer hidden states (within the bar), the K/V
written at every prompt position (within the bar of the oracle's, or one bf16 step of the element in a bf16
cache, at the closed-form offsets), nothing else
in the pool changed, and a decode continuing from the prefilled cache reproducing the oracle's tokens.
Sizes: the toy decoder in one chunk and in three (64 + 64 + 22 rows after a 5-position prefix), the
Qwen3-0.6B shape over 100 prompt tokens (two chunks) and the Llama-3-8B shape over 20 tokens after its
4,096-position prefix. The benchmark's size (a 2,048-token Qwen3-0.6B prompt) is in test_gpu_q06_full.py.
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


def margin(lg):
    s = np.sort(np.asarray(lg, np.float64))
    return (s[-1] - s[-2]) <= 2 * TOL * np.max(np.abs(s))


def kv_vals(a):
    a = np.asarray(a)
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def run_prefill(cfg, model, pool, slot, tokens, pos0):
    n = len(tokens)
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    lg = torch.full((cfg.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    hd = torch.full((cfg.n_layer * cfg.d,), float("nan"), dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, n))
    st = llmk.prefill(cfg, model, pool, slot, tokens, pos0, out, ws, lg, hd)
    assert st == llmk.OK, llmk.status_name(st)
    torch.cuda.synchronize()
    return host(out).tolist(), host(lg), host(hd)


def oracle_prefill(m, cache, tokens, pos0):
    """Teacher-forced oracle steps: greedy token and near-tie flag per position, last logits and hidden."""
    toks, ties, lg, hid = [], [], None, None
    for i, t in enumerate(tokens):
        lg, hid = m.forward_token(int(t), pos0 + i, cache, want_hidden=(i == len(tokens) - 1))
        toks.append(oracle.argmax(lg)[0])
        ties.append(margin(lg))
    return toks, ties, lg, hid


def check_tokens(got, want, ties, label):
    for i, (g, w, t) in enumerate(zip(got, want, ties)):
        if g != w:
            assert t, f"{label}: position {i}: token {g} != oracle {w}"
            say(f"{label}: position {i}: near-tie, gpu {g} oracle {w}")


def check_kv(s, pool, slot, cache, pos0, n, label):
    """K/V at the prompt positions of the slot, within the bar of the oracle's (TOL of the block's largest
    magnitude). A bf16 cache may also differ by one bf16 step of the element: both sides round an fp32 value
    that agrees within the bar, so a value near a rounding boundary lands on either side, and one step of a
    large element (2^-8 to 2^-7 of it) is more than the bar."""
    step = s.n_kv * s.head_dim
    base = slot * pool.capacity * step
    for l in range(s.n_layer):
        for which, buf, ref in (("k", pool.k[l], cache.k[l]), ("v", pool.v[l], cache.v[l])):
            got = host(buf)[base + pos0 * step: base + (pos0 + n) * step]
            g = kv_vals(got)
            w = kv_vals(np.asarray(ref[pos0:pos0 + n]).ravel())
            bar = TOL * np.max(np.abs(w))
            if got.dtype == np.uint16:
                mag = np.where(w != 0, np.abs(w), 1e-38)
                bar = np.maximum(bar, np.exp2(np.floor(np.log2(mag)) - 7))
            bad = np.abs(g - w) > bar
            assert not bad.any(), f"{label}: layer {l} {which}: {int(bad.sum())} elements off, e.g. {g[bad][:3]} vs {w[bad][:3]}"


TINY_BF16 = synth.TINY.with_(name="tiny-llama bf16 weights", w_dtype="bf16", max_seq=160)


@pytest.mark.parametrize("pos0,n", [(0, 10), (5, 150)])
def test_tiny_prefill_matches_oracle(pos0, n):
    s = TINY_BF16
    W = weights(s)
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 3, s.max_seq)
    m = oracle.Model(s, W)
    cache = m.new_cache(s.max_seq)
    if pos0 > 0:
        pre = [(k[:pos0], v[:pos0]) for k, v in synth.kv_prefix(s, pos0, seed=2)]
        loader.fill_prefix(pool, 1, pre)
        cache.fill_prefix(pre)
    before = {l: (host(pool.k[l]).copy(), host(pool.v[l]).copy()) for l in range(s.n_layer)}
    tokens = synth.prompt(n, s.vocab, stream=21).tolist()
    say(f"tiny prefill: {n} tokens from position {pos0}")
    got, g_lg, g_hd = run_prefill(cfg, model, pool, 1, tokens, pos0)
    want, ties, o_lg, o_hd = oracle_prefill(m, cache, tokens, pos0)
    check_tokens(got, want, ties, "tiny prefill")
    assert rel_err(g_lg, o_lg) <= TOL and rel_err(g_hd, o_hd) <= TOL
    check_kv(s, pool, 1, cache, pos0, n, "tiny prefill")
    assert int(pool.slot_len[1]) == pos0 + n
    # nothing outside the prompt positions of slot 1 changed
    step = s.n_kv * s.head_dim
    lo, hi = (1 * s.max_seq + pos0) * step, (1 * s.max_seq + pos0 + n) * step
    for l in range(s.n_layer):
        for now, was in ((host(pool.k[l]), before[l][0]), (host(pool.v[l]), before[l][1])):
            assert np.array_equal(np.delete(now, np.s_[lo:hi]), np.delete(was, np.s_[lo:hi]))
    # decoding on from the prefilled cache follows the oracle's greedy continuation
    k = min(4, s.max_seq - pos0 - n)
    dec = loader.Decoder(cfg, model, pool)
    toks = torch.zeros(k, dtype=torch.int32, device="cuda")
    assert dec.steps(got[-1], pos0 + n, k, toks, slot=1) == llmk.OK
    t, cont = want[-1], []
    for i in range(k):
        lg, _ = m.forward_token(t, pos0 + n + i, cache)
        t = oracle.argmax(lg)[0]
        cont.append(t)
    assert host(toks).tolist() == cont


@pytest.fixture(scope="module")
def q06():
    s = synth.Q06
    say("generating Qwen3-0.6B-shaped weights")
    W = weights(s)
    cfg = loader.config_from(s)
    return s, W, cfg, loader.upload_model(cfg, W)


def test_q06_prefill_two_chunks_matches_oracle(q06):
    s, W, cfg, model = q06
    n = 100
    pool = loader.new_pool(cfg, 2, 256)
    tokens = synth.prompt(n, s.vocab, stream=22).tolist()
    say(f"q06 prefill: {n} tokens")
    got, g_lg, g_hd = run_prefill(cfg, model, pool, 1, tokens, 0)
    m = oracle.Model(s, W)
    cache = m.new_cache(256)
    want, ties, o_lg, o_hd = oracle_prefill(m, cache, tokens, 0)
    check_tokens(got, want, ties, "q06 prefill")
    el, eh = rel_err(g_lg, o_lg), rel_err(g_hd, o_hd)
    say(f"q06 prefill: last logits rel err {el:.2e}, hidden {eh:.2e}")
    assert el <= TOL and eh <= TOL
    check_kv(s, pool, 1, cache, 0, n, "q06 prefill")


def test_llama8b_prefill_after_the_4096_prefix_matches_oracle():
    s = synth.L8B
    n_pre, n = 4096, 20
    say("generating 8B-shaped weights")
    W = weights(s)
    prefix = synth.kv_prefix(s, n_pre, seed=2)
    tokens = synth.prompt(n, s.vocab, stream=24).tolist()
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, n_pre + n)
    loader.fill_prefix(pool, 0, prefix)
    say(f"8B prefill: {n} tokens at positions {n_pre}..")
    got, g_lg, g_hd = run_prefill(cfg, model, pool, 0, tokens, n_pre)
    del model
    m = oracle.Model(s, W)
    cache = m.new_cache(n_pre + n)
    cache.fill_prefix(prefix)
    say("8B oracle steps")
    want, ties, o_lg, o_hd = oracle_prefill(m, cache, tokens, n_pre)
    check_tokens(got, want, ties, "8B prefill")
    el, eh = rel_err(g_lg, o_lg), rel_err(g_hd, o_hd)
    say(f"8B prefill: last logits rel err {el:.2e}, hidden {eh:.2e}")
    assert el <= TOL and eh <= TOL
    check_kv(s, pool, 0, cache, n_pre, n, "8B prefill")
