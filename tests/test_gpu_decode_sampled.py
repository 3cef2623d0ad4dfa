"""The sampled decode loop (llmk_decode_steps_sampled) against the oracle (GPU).

Each step's token is the oracle sampler's (temperature, top-k, top-p over the renormalised survivors, inverse
CDF at the step's uniform) applied to the oracle's logits of that step, the token fed back as the next input,
all inside the captured loop. The GPU samples from fp32 logits that agree with the oracle's within the bar, so a
step's token must equal the oracle's unless a decision of that step sits within 1e-4 of a boundary (the
uniform against a cumulative probability, the mass before a survivor against top-p, the k-th against the
(k+1)-th scaled logit); there the oracle takes the GPU's token as the next input, so every one of the steps is
compared on the same inputs, and all but those boundary steps must agree. Temperature 0 reproduces the greedy
loop. Sizes: the toy
decoder (a 40-entry vocabulary: the one-workgroup sampler), the Qwen3-0.6B shape (151,936 logits: the sliced
sampler) in the per-operation form, and the Llama-3-8B shape after its 4,096-position prefix in the persistent
form the benchmark times.
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import sampler
from tests.gpu_util import host, say, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402

EPS = 1e-4   # on scaled logits and on probabilities: far above the fp32-vs-fp64 logit differences


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def clear_of_boundaries(lg, T, k, p, u):
    if T == 0.0:
        s = np.sort(np.asarray(lg, np.float64))
        return s[-1] - s[-2] > EPS
    det = sampler.sample_detail(lg, T, k, p, u)
    z = np.asarray(lg, np.float64) / T
    order = det["order"]
    n = z.size
    kk = n if k <= 0 or k >= n else k
    zs = np.sort(z)[::-1]
    if kk < n and zs[kk - 1] - zs[kk] <= EPS:
        return False
    w = np.exp(z[order] - z[order[0]])
    prob = w / w.sum()
    before = np.concatenate(([0.0], np.cumsum(prob)[:-1]))
    if np.min(np.abs(before - p)) <= EPS:
        return False
    return np.min(np.abs(det["cdf"] - u)) > EPS


def run_case(s, step_path, n_pre, n, T, k, p, label):
    W = weights(s)
    prefix = synth.kv_prefix(s, n_pre, seed=2) if n_pre else None
    first = int(synth.prompt(1, s.vocab, stream=7)[0])
    draws = synth.draws((n,), seed=5, stream=31)
    cfg = loader.config_from(s, step_path=step_path)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, n_pre + n)
    if prefix:
        loader.fill_prefix(pool, 0, prefix)
    dec = loader.Decoder(cfg, model, pool)
    toks = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    d_draws = torch.from_numpy(np.asarray(draws, np.float32)).cuda()
    sws = llmk.workspace(max(llmk.sample_workspace_bytes(1, s.vocab, T, k), 16))
    say(f"{label}: {n} sampled steps (T {T}, top-k {k}, top-p {p}), form {llmk.decode_path(cfg)}")
    st = llmk.decode_steps_sampled(cfg, model, pool, 0, first, n_pre, n, T, k, p, d_draws, toks, dec.ws, sws)
    assert st == llmk.OK, llmk.status_name(st)
    torch.cuda.synchronize()
    got = host(toks).tolist()
    assert int(pool.slot_len[0]) == n_pre + n
    del model

    m = oracle.Model(s, W)
    c = m.new_cache(n_pre + n)
    if prefix:
        c.fill_prefix(prefix)
    t, equal, boundary = first, 0, []
    for i in range(n):
        lg, _ = m.forward_token(t, n_pre + i, c)
        u = float(draws[i])
        want = sampler.sample(lg, T, k, p, u)
        if got[i] != want:
            # a differing token must sit at a boundary; the oracle then follows the GPU's token
            assert not clear_of_boundaries(lg, T, k, p, u), f"{label}: step {i}: gpu {got[i]} oracle {want}"
            say(f"{label}: step {i} sits within {EPS} of a boundary: gpu {got[i]}, oracle {want}; the oracle follows")
            boundary.append(i)
        else:
            equal += 1
        t = got[i]
    say(f"{label}: {equal} of {n} steps equal, boundary steps {boundary}, tokens {got}")
    assert equal + len(boundary) == n and len(boundary) <= max(1, n // 8)
    return got


TINY_BF16 = synth.TINY.with_(name="tiny-llama bf16 weights", w_dtype="bf16")


@pytest.mark.parametrize("T,k,p", [(1.0, 0, 1.0), (0.7, 5, 0.9), (0.0, 0, 1.0)])
def test_tiny_sampled_loop_matches_oracle(T, k, p):
    run_case(TINY_BF16, llmk.STEP_PER_OP, 0, 12, T, k, p, "tiny")


def test_q06_sampled_loop_matches_oracle():
    run_case(synth.Q06, llmk.STEP_PER_OP, 32, 8, 0.8, 50, 0.9, "q06")


def test_llama8b_sampled_loop_persistent_matches_oracle():
    run_case(synth.L8B, llmk.STEP_AUTO, 4096, 4, 0.8, 50, 0.9, "8B")
