"""The Llama-3-8B-shaped decode step at full size against the oracle (MI355X only).

Workload: bf16 weights N(0, 0.02), unit gains, RoPE base 5e5, a bf16 K/V pool whose positions
0..4095 hold seeded N(0, 1) values (the same bytes in the oracle's cache), then greedy steps from
position 4096 through the same launch configuration the benchmark times (decode_steps: one captured
step replayed with device token feedback). Both forms of the step run: the persistent one-kernel step
(what the library picks for this shape) and one kernel per operation.
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

N_PRE = 4096
N_STEPS = 3


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def l8b():
    """Weights, prefix, first token, and the oracle's tokens / logits / hidden states at 4096.."""
    s = synth.L8B
    say("generating 8B-shaped weights")
    W = synth.model(s, seed=0)
    prefix = synth.kv_prefix(s, N_PRE, seed=2)
    first = int(synth.prompt(1, s.vocab, stream=7)[0])
    say("oracle: steps at positions 4096..")
    m = oracle.Model(s, W)
    c = m.new_cache(N_PRE + N_STEPS)
    c.fill_prefix(prefix)
    o_tokens, o_logits, o_hidden = [], [], []
    t = first
    for i in range(N_STEPS):
        lg, hid = m.forward_token(t, N_PRE + i, c, want_hidden=True)
        o_logits.append(lg)
        o_hidden.append(hid)
        t = oracle.argmax(lg)[0]
        o_tokens.append(t)
    say(f"oracle tokens {o_tokens}")
    return s, W, prefix, first, c, o_tokens, o_logits, o_hidden


def test_library_picks_the_persistent_step_for_the_8b_shape():
    cfg = loader.config_from(synth.L8B)
    assert llmk.decode_path(cfg) == llmk.STEP_PERSISTENT
    assert llmk.decode_path(loader.config_from(synth.L8B, step_path=llmk.STEP_PER_OP)) == llmk.STEP_PER_OP


@pytest.mark.parametrize("step_path", [llmk.STEP_AUTO, llmk.STEP_PER_OP])
def test_llama8b_full_size_matches_oracle(l8b, step_path):
    s, W, prefix, first, c, o_tokens, o_logits, o_hidden = l8b
    say(f"GPU ({'library choice' if step_path == llmk.STEP_AUTO else 'per-op'}): upload and decode_steps")
    cfg = loader.config_from(s, step_path=step_path)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, s.max_seq)
    loader.fill_prefix(pool, 0, prefix)
    dec = loader.Decoder(cfg, model, pool)
    toks = torch.zeros(N_STEPS, dtype=torch.int32, device="cuda")
    assert dec.steps(first, N_PRE, N_STEPS, toks) == llmk.OK
    gpu_free = host(toks).tolist()
    say(f"gpu tokens {gpu_free}")

    # teacher-forced single steps on a second slot-pool (same prefix) for logits and hidden states
    pool2 = loader.new_pool(cfg, 1, N_PRE + N_STEPS)
    loader.fill_prefix(pool2, 0, prefix)
    dec2 = loader.Decoder(cfg, model, pool2)
    ins = [first] + o_tokens[:-1]
    for i, tin in enumerate(ins):
        lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
        hid = torch.empty(s.n_layer * s.d, dtype=torch.float32, device="cuda")
        assert dec2.step(tin, N_PRE + i, 0, lg, hid) == llmk.OK
        torch.cuda.synchronize()
        el = rel_err(host(lg), o_logits[i])
        eh = rel_err(host(hid).reshape(s.n_layer, s.d), o_hidden[i])
        say(f"step {i}: logits err {el:.2e} hidden err {eh:.2e}")
        assert el <= TOL and eh <= TOL
        assert int(host(dec2.token_out)[0]) == o_tokens[i]
    assert gpu_free == o_tokens
    # the K/V written at 4096.. sits at the closed-form offsets, bf16 of the oracle's values
    for l in (0, s.n_layer - 1):
        got = host(pool2.slot_view(l, 0, "k"))[N_PRE:N_PRE + N_STEPS]
        ref = oracle.bf16_to_f64(c.k[l][N_PRE:N_PRE + N_STEPS])
        assert rel_err(oracle.bf16_to_f64(got), ref) <= TOL
        assert np.array_equal(host(pool2.slot_view(l, 0, "k"))[:N_PRE], prefix[l][0])

    if step_path == llmk.STEP_AUTO:
        # the timing aid for the persistent kernel leaves the slot as one ordinary step at 4096 does
        pool2.slot_len[0] = N_PRE
        st, ms = llmk.decode_kernel_time(cfg, model, pool2, 0, first, N_PRE, llmk.STEP_KERNEL, 3, dec2.token_out,
                                         dec2.ws)
        assert st == llmk.OK and ms > 0
        assert int(host(dec2.token_out)[0]) == o_tokens[0]
        assert pool2.slot_len[0] == N_PRE + 1
