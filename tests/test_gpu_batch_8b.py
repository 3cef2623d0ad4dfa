"""The batched decode step at full size: Llama-3-8B shape, 64 sequences with seeded contexts uniform in
512..8192 (MI355X only), in the launch configuration the batched benchmark times.

The GPU runs all 64 rows; the oracle computes sampled rows one by one (the shortest and the longest
context, and two more), each on its own cache filled with the same K/V bytes.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, host, rel_err, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402

B = 64
CTX_LO, CTX_HI = 512, 8192


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def near_tie(logits, tol=TOL):
    s = np.sort(np.asarray(logits, np.float64))
    return (s[-1] - s[-2]) <= 2 * tol * np.max(np.abs(s))


def test_llama8b_batch64_matches_oracle_on_sampled_rows():
    s = synth.L8B.with_(name="llama-3-8b-shaped bf16, batched", max_seq=CTX_HI + 8)
    say("generating 8B-shaped weights and the K/V source")
    W = synth.model(s, seed=0)
    ctxs = synth.ragged_contexts(B, CTX_LO, CTX_HI, seed=3).tolist()
    src = synth.kv_prefix(s, CTX_HI + synth.slot_window(B - 1), seed=2)
    tokens = synth.prompt(B, s.vocab, stream=13).tolist()
    slots = [(7 * r) % B for r in range(B)]          # rows map to slots out of order

    say("GPU: upload, fill 64 slots, one batched step")
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, B, s.max_seq)
    src_dev = loader.upload_kv_source(src)
    for r in range(B):
        loader.fill_prefix_window(pool, slots[r], src_dev, synth.slot_window(r), ctxs[r])
    del src_dev
    dec = loader.BatchDecoder(cfg, model, pool, B)
    lg = torch.empty(B * s.vocab, dtype=torch.float32, device="cuda")
    hd = torch.empty(B * s.n_layer * s.d, dtype=torch.float32, device="cuda")
    assert dec.step(slots, tokens, ctxs, lg, hd) == llmk.OK
    torch.cuda.synchronize()
    g_tok = host(dec.tokens_out).tolist()
    g_lg = host(lg).reshape(B, s.vocab)
    g_hd = host(hd).reshape(B, s.n_layer, s.d)
    n = 2
    out = torch.zeros(n * B, dtype=torch.int32, device="cuda")
    assert dec.steps(slots, g_tok, [c + 1 for c in ctxs], n, out) == llmk.OK
    g_more = host(out).reshape(n, B)

    rows = sorted({int(np.argmin(ctxs)), int(np.argmax(ctxs)), 0, 37})
    m = oracle.Model(s, W)
    for r in rows:
        say(f"oracle: row {r} (slot {slots[r]}, context {ctxs[r]})")
        c = m.new_cache(ctxs[r] + 1 + n)
        st = synth.slot_window(r)
        c.fill_prefix([(k[st:st + ctxs[r]], v[st:st + ctxs[r]]) for k, v in src])
        o_lg, o_hd = m.forward_token(tokens[r], ctxs[r], c, want_hidden=True)
        el, eh = rel_err(g_lg[r], o_lg), rel_err(g_hd[r], o_hd)
        say(f"row {r}: logits err {el:.2e} hidden err {eh:.2e}")
        assert el <= TOL and eh <= TOL
        want = oracle.argmax(o_lg)[0]
        if g_tok[r] != want:
            assert near_tie(o_lg), f"row {r}: token {g_tok[r]} != oracle {want}"
            continue
        t = want
        for i in range(n):
            o2, _ = m.forward_token(t, ctxs[r] + 1 + i, c)
            t = oracle.argmax(o2)[0]
            assert int(g_more[i, r]) == t, f"row {r} step {i + 1}"
        del c
