"""The Qwen3-0.6B-shaped workload at its full size against the oracle (MI355X only).

bf16 weights N(0, 0.02), fp32 K/V, RoPE base 1e6: a seeded 2,048-token prompt runs through the library's
prefill (chunks of rows through the layers), then 128 greedy decode steps at positions 2,048..2,175.

Prefill: the oracle's chunked forward over the same 2,048 tokens (its definition is the token-by-token step,
to which the chunked form is pinned). At every one of the 2,048 positions the GPU's greedy token equals the
oracle's (or the oracle's top two are within the bar, reported); the last position's logits and hidden states
and the K/V of every position and layer are within 2e-3.

Decode: the GPU runs free from the prefill's last greedy token, one call per step (logits and hidden states
kept) and, from a second identical prefill, as graph replays with device token feedback; the two give the
same tokens. The oracle, teacher-forced on the GPU's inputs from its own prefilled cache, agrees at all 128
steps: token, logits and hidden states as above.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import chunk
from tests.gpu_util import TOL, host, rel_err, say, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402

N_PROMPT = 2048
N_STEPS = 128


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def near_tie(logits, tol=TOL):
    s = np.sort(np.asarray(logits, np.float64))
    return (s[-1] - s[-2]) <= 2 * tol * np.max(np.abs(s))


def prefill(cfg, model, pool, slot, tokens):
    n = len(tokens)
    out = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    lg = torch.full((cfg.vocab,), float("nan"), dtype=torch.float32, device="cuda")
    hd = torch.full((cfg.n_layer * cfg.d,), float("nan"), dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, n))
    st = llmk.prefill(cfg, model, pool, slot, tokens, 0, out, ws, lg, hd)
    assert st == llmk.OK, llmk.status_name(st)
    torch.cuda.synchronize()
    return host(out).tolist(), host(lg), host(hd).reshape(cfg.n_layer, cfg.d)


def test_q06_2048_prefill_then_128_steps_match_oracle():
    s = synth.Q06
    say("generating Qwen3-0.6B-shaped weights")
    W = weights(s)
    prompt = synth.prompt(N_PROMPT, s.vocab, stream=23).tolist()
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 2, s.max_seq)
    say("GPU: 2,048-token prefill into slots 0 and 1")
    p_tok, p_lg, p_hd = prefill(cfg, model, pool, 0, prompt)
    p_tok1, _, _ = prefill(cfg, model, pool, 1, prompt)
    assert p_tok1 == p_tok
    dec = loader.Decoder(cfg, model, pool)
    fed, toks = [p_tok[-1]], []
    g_lg = np.empty((N_STEPS, s.vocab), np.float32)
    g_hd = np.empty((N_STEPS, s.n_layer, s.d), np.float32)
    lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    hd = torch.empty(s.n_layer * s.d, dtype=torch.float32, device="cuda")
    say("GPU: 128 decode steps, one call each")
    for i in range(N_STEPS):
        assert dec.step(fed[i], N_PROMPT + i, 0, lg, hd) == llmk.OK
        torch.cuda.synchronize()
        toks.append(int(host(dec.token_out)[0]))
        g_lg[i] = host(lg)
        g_hd[i] = host(hd).reshape(s.n_layer, s.d)
        if i + 1 < N_STEPS:
            fed.append(toks[-1])
    out = torch.zeros(N_STEPS, dtype=torch.int32, device="cuda")
    say("GPU: the same 128 steps as graph replays on slot 1")
    assert dec.steps(p_tok[-1], N_PROMPT, N_STEPS, out, slot=1) == llmk.OK
    assert host(out).tolist() == toks
    pool_k = [host(pool.slot_view(l, 0, "k"))[:N_PROMPT] for l in range(s.n_layer)]
    pool_v = [host(pool.slot_view(l, 0, "v"))[:N_PROMPT] for l in range(s.n_layer)]
    del model, pool, dec
    torch.cuda.empty_cache()

    say("oracle: the prompt as one chunk")
    m = oracle.Model(s, W)
    cache = m.new_cache(N_PROMPT + N_STEPS)
    w = chunk.Weights(s, W)
    o_lg, o_hd = chunk.forward_chunk(s, w, prompt, 0, cache)
    ties = []
    for i in range(N_PROMPT):
        want = oracle.argmax(o_lg[i])[0]
        if p_tok[i] != want:
            assert near_tie(o_lg[i]), f"prefill position {i}: token {p_tok[i]} != oracle {want}"
            ties.append(i)
    el, eh = rel_err(p_lg, o_lg[-1]), rel_err(p_hd, o_hd[-1])
    say(f"prefill: last logits err {el:.2e}, hidden err {eh:.2e}; tolerance ties at positions {ties} (reported)")
    assert el <= TOL and eh <= TOL
    for l in range(s.n_layer):
        for which, got, ref in (("k", pool_k[l], cache.k[l]), ("v", pool_v[l], cache.v[l])):
            e = rel_err(got, ref[:N_PROMPT])
            assert e <= TOL, f"prefill K/V layer {l} {which}: {e:.3e}"
    del o_lg, o_hd

    say("oracle: the 128 GPU decode inputs teacher-forced, one chunk")
    d_lg, d_hd = chunk.forward_chunk(s, w, fed, N_PROMPT, cache)
    ties, worst_l, worst_h = [], 0.0, 0.0
    for i in range(N_STEPS):
        el, eh = rel_err(g_lg[i], d_lg[i]), rel_err(g_hd[i], d_hd[i])
        worst_l, worst_h = max(worst_l, el), max(worst_h, eh)
        assert el <= TOL, f"decode step {i}: logits rel err {el:.3e}"
        assert eh <= TOL, f"decode step {i}: hidden rel err {eh:.3e}"
        want = oracle.argmax(d_lg[i])[0]
        if toks[i] != want:
            assert near_tie(d_lg[i]), f"decode step {i}: token {toks[i]} != oracle {want}"
            ties.append(i)
    say(f"decode: worst logits err {worst_l:.2e}, worst hidden err {worst_h:.2e}; tolerance ties at {ties}")
