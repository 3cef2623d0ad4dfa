"""The Llama-3-8B-shaped decode at its full size and length against the oracle (MI355X only).

Workload: bf16 weights N(0, 0.02), unit gains, RoPE base 5e5, a bf16 K/V pool whose positions 0..4095 hold
seeded N(0, 1) values (the same bytes in the oracle's cache), then 256 greedy steps at positions 4096..4351.

The GPU runs free: the step at position 4096 + i consumes the greedy token of step i - 1. It runs once one
call per step (keeping every step's logits and per-layer hidden states) and once as the benchmark times it
(one captured step replayed 256 times with device token feedback); both must give the same tokens. The
oracle is then teacher-forced on the GPU's inputs (its chunked form over the 256 rows), and at every step:
the GPU's token equals the oracle's greedy token (or the oracle's top two are within the bar, reported),
and the logits and hidden states are within 2e-3. The 256 steps cross 4 attention tiles of 64 positions
and every context-part boundary the split uses between 4,097 and 4,352 positions. The one-kernel-per-
operation form runs the same inputs against the same oracle rows.
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

N_PRE = 4096
N_STEPS = 256


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def near_tie(logits, tol=TOL):
    s = np.sort(np.asarray(logits, np.float64))
    return (s[-1] - s[-2]) <= 2 * tol * np.max(np.abs(s))


def gpu_loop(dec, s, inputs, feed_own=True):
    """One decode_step call per step from position N_PRE; with feed_own the next input is the step's own
    greedy token (inputs holds only the first). Returns (inputs fed, tokens, logits [n][V], hidden [n][L][d])."""
    n = N_STEPS
    fed, toks = [int(inputs[0])], []
    lg_all = np.empty((n, s.vocab), np.float32)
    hid_all = np.empty((n, s.n_layer, s.d), np.float32)
    lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
    hid = torch.empty(s.n_layer * s.d, dtype=torch.float32, device="cuda")
    for i in range(n):
        assert dec.step(fed[i], N_PRE + i, 0, lg, hid) == llmk.OK
        torch.cuda.synchronize()
        toks.append(int(host(dec.token_out)[0]))
        lg_all[i] = host(lg)
        hid_all[i] = host(hid).reshape(s.n_layer, s.d)
        if i + 1 < n:
            fed.append(toks[-1] if feed_own else int(inputs[i + 1]))
    return fed, toks, lg_all, hid_all


def compare(label, toks, lg, hid, o_lg, o_hid):
    worst_l = worst_h = 0.0
    ties = []
    for i in range(N_STEPS):
        el, eh = rel_err(lg[i], o_lg[i]), rel_err(hid[i], o_hid[i])
        worst_l, worst_h = max(worst_l, el), max(worst_h, eh)
        assert el <= TOL, f"{label} step {i}: logits rel err {el:.3e}"
        assert eh <= TOL, f"{label} step {i}: hidden rel err {eh:.3e}"
        want = oracle.argmax(o_lg[i])[0]
        if toks[i] != want:
            assert near_tie(o_lg[i]), f"{label} step {i}: token {toks[i]} != oracle {want}"
            ties.append(i)
    say(f"{label}: {N_STEPS} steps, worst logits err {worst_l:.2e}, worst hidden err {worst_h:.2e}, "
        f"tolerance ties at steps {ties} (reported)")


@pytest.fixture(scope="module")
def run8b():
    """The persistent form's free run (per-call and graph-replayed) and the oracle teacher-forced on it."""
    s = synth.L8B
    say("generating 8B-shaped weights and the 4,096-position K/V prefix")
    W = weights(s)
    prefix = synth.kv_prefix(s, N_PRE, seed=2)
    first = int(synth.prompt(1, s.vocab, stream=7)[0])
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, s.max_seq)
    loader.fill_prefix(pool, 0, prefix)
    dec = loader.Decoder(cfg, model, pool)
    say("GPU: 256 steps, one call each")
    fed, toks, lg, hid = gpu_loop(dec, s, [first])
    say(f"GPU tokens {toks[:12]} ...")
    pool2 = loader.new_pool(cfg, 1, s.max_seq)
    loader.fill_prefix(pool2, 0, prefix)
    dec2 = loader.Decoder(cfg, model, pool2)
    out = torch.zeros(N_STEPS, dtype=torch.int32, device="cuda")
    say("GPU: 256 steps as graph replays (the benchmark's launch configuration)")
    assert dec2.steps(first, N_PRE, N_STEPS, out) == llmk.OK
    graph_toks = host(out).tolist()
    say("oracle: the 256 GPU inputs teacher-forced, one chunk")
    m = oracle.Model(s, W)
    cache = m.new_cache(N_PRE + N_STEPS)
    cache.fill_prefix(prefix)
    o_lg, o_hid = chunk.forward_chunk(s, chunk.Weights(s, W), fed, N_PRE, cache)
    yield dict(s=s, W=W, prefix=prefix, cfg=cfg, model=model, pool=pool, fed=fed, toks=toks, lg=lg, hid=hid,
               graph_toks=graph_toks, cache=cache, o_lg=o_lg, o_hid=o_hid, dec=dec)
    del model, pool, pool2, dec, dec2
    torch.cuda.empty_cache()


def test_library_picks_the_persistent_step_for_the_8b_shape():
    cfg = loader.config_from(synth.L8B)
    assert llmk.decode_path(cfg) == llmk.STEP_PERSISTENT
    assert llmk.decode_path(loader.config_from(synth.L8B, step_path=llmk.STEP_PER_OP)) == llmk.STEP_PER_OP


def test_llama8b_256_steps_match_oracle(run8b):
    r = run8b
    s = r["s"]
    assert r["graph_toks"] == r["toks"], "graph replay and per-call steps disagree"
    compare("8B persistent", r["toks"], r["lg"], r["hid"], r["o_lg"], r["o_hid"])
    # the K/V the 256 steps appended, every layer: bf16 of the oracle's values (within the bar, or one bf16
    # step of the element), at the closed-form offsets; the prefix untouched
    for l in range(s.n_layer):
        for which, ref in (("k", r["cache"].k[l]), ("v", r["cache"].v[l])):
            got = host(r["pool"].slot_view(l, 0, which))
            g = oracle.widen(got[N_PRE:N_PRE + N_STEPS])
            w = oracle.widen(ref[N_PRE:N_PRE + N_STEPS])
            mag = np.where(w != 0, np.abs(w), 1e-38)
            bar = np.maximum(TOL * np.max(np.abs(w)), np.exp2(np.floor(np.log2(mag)) - 7))
            assert not (np.abs(g - w) > bar).any(), f"layer {l} {which}"
            assert np.array_equal(got[:N_PRE], r["prefix"][l][0 if which == "k" else 1])


def test_llama8b_per_operation_form_matches_oracle(run8b):
    r = run8b
    s = r["s"]
    cfg = loader.config_from(s, step_path=llmk.STEP_PER_OP)
    pool = loader.new_pool(cfg, 1, s.max_seq)
    loader.fill_prefix(pool, 0, r["prefix"])
    dec = loader.Decoder(cfg, r["model"], pool)
    say("GPU per-operation form: the same 256 inputs")
    fed, toks, lg, hid = gpu_loop(dec, s, r["fed"], feed_own=False)
    assert fed == r["fed"]
    compare("8B per-op", toks, lg, hid, r["o_lg"], r["o_hid"])


def test_llama8b_step_kernel_timing_aid_leaves_an_ordinary_step(run8b):
    r = run8b
    s = r["s"]
    pool = loader.new_pool(r["cfg"], 1, s.max_seq)
    loader.fill_prefix(pool, 0, r["prefix"])
    dec = loader.Decoder(r["cfg"], r["model"], pool)
    st, ms = llmk.decode_kernel_time(r["cfg"], r["model"], pool, 0, r["fed"][0], N_PRE, llmk.STEP_KERNEL, 3,
                                     dec.token_out, dec.ws)
    assert st == llmk.OK and ms > 0
    assert int(host(dec.token_out)[0]) == r["toks"][0]
    assert pool.slot_len[0] == N_PRE + 1
