"""Parity of the sampling exit (llmk_sample) with the oracle's sampler, through the C-ABI (GPU).

Workloads: Llama-3-vocabulary rows (128,256 logits, N(0, 3)) at batch 1 and 64, ragged small rows, and
planted structure: ties across the top-k cut (more ties than survivors, spread over the row), all-equal
rows, signed zeros, NaN and infinities, and draws at 0, just below 1, at 1 and below 0.

The bar: the token is bit-exact, except where the oracle itself sits within 1e-9 of a boundary (a
cumulative probability at the draw, or the mass before a survivor at top_p): both sides compute those
sums in fp64 in different orders, so there the token must be one the oracle gives with the draw or top_p
moved by 1e-9 either way. Temperature, top_p and the draws are fp32 values, handed to both sides exactly.
"""
import numpy as np
import pytest

import synth
from oracle.sampler import sample_detail
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")

V = 128256
EPS = 1e-9


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def f32(v) -> float:
    return float(np.float32(v))


def run_sample(logits, t, k, p, u):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    rows, n = logits.shape
    u = np.ascontiguousarray(u, dtype=np.float32).ravel()
    assert u.size == rows
    lg, ud = dev(logits.ravel()), dev(u)
    tok = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    need = llmk.sample_workspace_bytes(rows, n, f32(t), k)
    assert need >= 0, need
    ws = llmk.workspace(need) if need > 0 else None
    st = llmk.sample(lg, rows, n, f32(t), k, f32(p), ud, tok, ws)
    assert st == llmk.OK, st
    torch.cuda.synchronize()
    return host(tok)


def acceptable(row, t, k, p, u) -> set:
    """The oracle's token, plus its tokens with the draw or top_p moved by EPS where that changes them."""
    t, p, u = f32(t), f32(p), f32(u)
    out = {sample_detail(row, t, k, p, u)["token"]}
    for du in (-EPS, 0.0, EPS):
        for dp in (-EPS, 0.0, EPS):
            pp = min(1.0, max(p + dp, 1e-12))
            out.add(sample_detail(row, t, k, pp, u + du)["token"])
    return out


def check_rows(logits, t, k, p, u, tag):
    say(f"sample {tag}: rows={logits.shape[0]} n={logits.shape[1]} T={t} k={k} p={p}")
    got = run_sample(logits, t, k, p, u)
    exact = 0
    for r in range(logits.shape[0]):
        ref = sample_detail(logits[r], f32(t), k, f32(p), f32(u[r]))["token"]
        if got[r] == ref:
            exact += 1
            continue
        ok = acceptable(logits[r], t, k, p, u[r])
        assert got[r] in ok, (tag, r, int(got[r]), ref, sorted(ok))
    return exact


GRID = [(0.0, 50, 0.9), (0.6, 50, 0.9), (1.0, 1, 1.0), (1.0, 20, 0.5), (1.0, 1024, 1.0), (1.7, 1024, 0.95),
        (0.8, 400, 0.99), (3.0, 7, 0.3)]


@pytest.mark.parametrize("t,k,p", GRID)
def test_vocab_rows_match_the_oracle(t, k, p):
    rows = 8
    logits = synth.normal((rows, V), 500, 0, 3.0)
    u = synth.draws((rows,), 501, int(1000 * t) + k)
    u[0], u[1] = 0.0, np.nextafter(np.float32(1.0), np.float32(0.0))
    exact = check_rows(logits, t, k, p, u, "vocab")
    assert exact >= rows - 1


def test_batch_of_64_vocab_rows():
    logits = synth.normal((64, V), 510, 0, 3.0)
    u = synth.draws((64,), 511, 0)
    assert check_rows(logits, 0.9, 50, 0.95, u, "batch64") >= 63


@pytest.mark.parametrize("k,n_ties", [(50, 3000), (50, 300), (300, 3000)])
def test_draw_sweep_recovers_the_survivor_order(k, n_ties):
    # one row repeated with draws at the middle of each survivor's interval: every survivor is hit once,
    # so the tokens spell the survivor order (values, then the lower index among ties); k 50 takes the
    # wave slices (300 ties: few enough candidates above the slice-maximum floor to rank directly; 3000: the
    # full selection), 300 the block slices
    row = synth.normal((V,), 520, 0, 3.0)
    order = np.lexsort((np.arange(V), -row.astype(np.float64)))
    cut = float(row[order[30]])
    row[synth.ints((n_ties,), 0, V - 1, 521, 0)] = cut      # ties at the cut, more than survive
    d = sample_detail(row, 1.0, k, 1.0, 0.0)
    mids = np.concatenate(([0.0], d["cdf"][:-1])) + np.diff(np.concatenate(([0.0], d["cdf"]))) / 2
    u = mids.astype(np.float32)
    logits = np.repeat(row[None, :], k, axis=0)
    got = run_sample(logits, 1.0, k, 1.0, u)
    assert list(got) == list(d["order"][:k])
    assert check_rows(logits, 1.0, k, 1.0, u, "sweep") == k


def test_rows_longer_than_the_slices_take_the_one_workgroup_form():
    # a Qwen-sized vocabulary at top-k 1024 does not fit 8 slices of 16,384 logits
    n = 151936
    assert llmk.sample_workspace_bytes(2, n, 1.0, 1024) == 0
    logits = synth.normal((2, n), 570, 0, 3.0)
    logits[1, synth.ints((500,), 0, n - 1, 571, 0)] = float(np.sort(logits[1])[-900])   # ties at the cut
    u = synth.draws((2,), 572, 0)
    for t, k, p in [(1.0, 1024, 1.0), (0.7, 1024, 0.9), (1.0, 1000, 0.5)]:
        check_rows(logits, t, k, p, u, "wide")


@pytest.mark.parametrize("k", [50, 500])
def test_all_equal_vocab_rows_take_the_lowest_indices(k):
    # every slice holds more ties than survivors: each keeps its lowest indices, the merge the lowest overall
    logits = np.full((k, V), -1.5, np.float32)
    u = ((np.arange(k) + 0.5) / k).astype(np.float32)
    assert list(run_sample(logits, 1.0, k, 1.0, u)) == list(range(k))


def test_equal_logits_are_the_uniform_law_over_the_lowest_indices():
    n, k = 5000, 1024
    logits = np.full((k, n), 0.25, np.float32)
    u = ((np.arange(k) + 0.5) / k).astype(np.float32)
    got = run_sample(logits, 1.0, k, 1.0, u)
    assert list(got) == list(range(k))                      # token = floor(k u) over indices 0..k-1


def test_small_and_ragged_rows():
    for n in (1, 2, 3, 7, 63, 64, 65, 1023, 1024, 1025, 4099):
        logits = synth.normal((5, n), 530 + n, 0, 2.0)
        u = synth.draws((5,), 531, n)
        for t, k, p in [(1.0, 0, 1.0), (0.5, 3, 0.8), (0.0, 0, 1.0), (2.0, 2000, 0.6)]:
            if t > 0 and (n if k <= 0 or k >= n else k) > 1024:
                continue                                    # more survivors than the sampler holds
            check_rows(logits, t, k, p, u, f"n={n}")


def test_signed_zero_nan_and_infinities():
    rows = np.full((6, 300), -2.0, np.float32)
    rows[0, [10, 20]] = [-0.0, 0.0]                         # equal: the lower index comes first
    rows[1, [10, 20]] = [0.0, -0.0]
    rows[2, [5, 100, 200]] = [np.nan, 1.0, np.nan]          # NaN counts as -inf
    rows[3, :] = np.nan                                     # nothing finite: the first survivor, index 0
    rows[4, [7, 9]] = [np.inf, np.inf]                      # +inf on top: the first survivor
    rows[5, :] = -np.inf
    rows[5, 250] = -1e30
    for t, k, p in [(1.0, 4, 1.0), (0.0, 0, 1.0), (0.3, 300, 0.5)]:
        for u0 in (0.0, 0.4, 0.99):
            u = np.full(6, u0, np.float32)
            check_rows(rows, t, k, p, u, f"edges u={u0}")
    got = run_sample(rows[:2], 1.0, 2, 1.0, np.array([0.0, 0.0], np.float32))
    assert list(got) == [10, 10]


def test_draws_outside_the_unit_interval():
    row = synth.normal((1, 1000), 540, 0, 1.0)
    d = sample_detail(row[0], 1.0, 10, 0.9, 0.0)
    first, last = int(d["order"][0]), int(d["order"][d["kept"] - 1])
    for u, want in [(-0.5, first), (float("nan"), first), (1.0, last), (7.0, last)]:
        assert run_sample(row, 1.0, 10, 0.9, np.array([u], np.float32))[0] == want, u


def test_same_inputs_same_tokens():
    logits = synth.normal((16, V), 550, 0, 3.0)
    u = synth.draws((16,), 551, 0)
    a = run_sample(logits, 1.1, 200, 0.97, u)
    b = run_sample(logits, 1.1, 200, 0.97, u)
    assert np.array_equal(a, b)


def test_frequencies_follow_the_kept_distribution():
    # 4096 draws on the grid (i + 0.5) / 4096 over one 9-logit row: counts = 4096 x the kept probabilities
    row = synth.normal((9,), 560, 0, 1.5)
    m = 4096
    u = ((np.arange(m) + 0.5) / m).astype(np.float32)
    got = run_sample(np.repeat(row[None, :], m, axis=0), 0.7, 5, 0.9, u)
    d = sample_detail(row, f32(0.7), 5, f32(0.9), 0.0)
    kept = d["order"][:d["kept"]]
    q = np.diff(np.concatenate(([0.0], d["cdf"])))
    for tok, pr in zip(kept, q):
        assert abs(np.count_nonzero(got == tok) - m * pr) <= 1.0
    assert set(np.unique(got)) <= set(int(i) for i in kept)
