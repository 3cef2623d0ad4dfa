"""Pins of the oracle's sampler against closed forms, the tie rule the decode-ops page states, the
HuggingFace top-p rule on hand-worked masses, and an independent brute-force distribution (CPU only)."""
import math

import numpy as np
import pytest
import scipy.special

from oracle import contract
from oracle.sampler import sample, sample_detail

RNG = np.random.default_rng(77)


def test_temperature_zero_is_greedy_with_ties_to_the_lower_index():
    assert sample([1.0, 3.0, 3.0, 2.0], 0.0, 0, 1.0, 0.99) == 1
    assert sample([5.0, 5.0], 0.0, 50, 0.9, 0.5) == 0


def test_top_k_one_is_the_argmax_for_any_draw():
    x = RNG.standard_normal(1000)
    for u in (0.0, 0.3, 0.999999):
        assert sample(x, 0.8, 1, 0.95, u) == int(np.argmax(x))


def test_zero_draw_takes_the_first_survivor():
    x = RNG.standard_normal(500)
    assert sample(x, 1.3, 40, 0.9, 0.0) == int(np.argmax(x))


def test_two_tokens_closed_form():
    # probabilities 1/4 and 3/4; descending order puts token 1 first
    x = [0.0, math.log(3.0)]
    assert sample(x, 1.0, 0, 1.0, 0.0) == 1
    assert sample(x, 1.0, 0, 1.0, 0.7499) == 1
    assert sample(x, 1.0, 0, 1.0, 0.75) == 0          # the CDF at token 1 is exactly 0.75: not above it
    assert sample(x, 1.0, 0, 1.0, 0.9) == 0


def test_temperature_scales_the_logits():
    # logits [0, 1] at T = 0.5: probabilities proportional to [1, e^2]
    p1 = math.exp(2.0) / (1.0 + math.exp(2.0))
    assert sample([0.0, 1.0], 0.5, 0, 1.0, p1 - 1e-9) == 1
    assert sample([0.0, 1.0], 0.5, 0, 1.0, p1 + 1e-9) == 0


def test_equal_logits_give_the_inverse_cdf_of_the_uniform_law():
    # ten equal logits: the order is the index order and token = floor(10 u)
    for u in (0.0, 0.05, 0.15, 0.55, 0.95, 0.99):
        assert sample(np.zeros(10), 1.0, 0, 1.0, u) == int(math.floor(10 * u))


@pytest.mark.parametrize("p,kept", [(0.49999, 1), (0.50001, 2), (0.79999, 2), (0.80001, 3), (1.0, 3)])
def test_top_p_keeps_while_the_mass_before_is_below_p(p, kept):
    # masses 0.5, 0.3, 0.2 in descending order: the mass before each is 0, 0.5, 0.8 (p is kept off those
    # boundaries, where fp64 rounding of the masses decides)
    d = sample_detail(np.log([0.2, 0.5, 0.3]), 1.0, 0, p, 0.0)
    assert d["kept"] == kept
    assert list(d["order"][:3]) == [1, 2, 0]


def test_top_p_renormalises_over_the_kept():
    # p just under 0.8 keeps masses 0.5 and 0.3 -> 0.625 and 0.375
    x = np.log([0.2, 0.5, 0.3])
    assert sample(x, 1.0, 0, 0.79999, 0.6249) == 1
    assert sample(x, 1.0, 0, 0.79999, 0.6251) == 2
    assert sample(x, 1.0, 0, 0.79999, 0.9999) == 2


def test_top_k_ties_go_to_the_lower_index():
    # values 2, 5, 5, 1: with k = 2 the survivors are tokens 1 and 2, in that order
    d = sample_detail([2.0, 5.0, 5.0, 1.0], 1.0, 2, 1.0, 0.0)
    assert list(d["order"]) == [1, 2]
    assert sample([2.0, 5.0, 5.0, 1.0], 1.0, 2, 1.0, 0.49) == 1
    assert sample([2.0, 5.0, 5.0, 1.0], 1.0, 2, 1.0, 0.51) == 2


def test_nan_counts_as_minus_infinity():
    assert sample([float("nan"), 1.0, 0.0], 1.0, 0, 1.0, 0.0) == 1
    d = sample_detail([float("nan"), 1.0, 0.0], 1.0, 0, 1.0, 0.0)
    assert 0 not in list(d["order"][:d["kept"]]) or d["cdf"][-1] == d["cdf"][-2]


def _brute_force_probs(x, t, k, p):
    """Independent reading: sort with Python's sorted on (-value, index), cut, softmax with scipy."""
    z = [v / t for v in x]
    idx = sorted(range(len(z)), key=lambda i: (-z[i], i))
    if 0 < k < len(z):
        idx = idx[:k]
    probs = scipy.special.softmax(np.array([z[i] for i in idx]))
    keep, acc = [], 0.0
    for i, pr in zip(idx, probs):
        if acc < p:
            keep.append(i)
        acc += pr
    q = scipy.special.softmax(np.array([z[i] for i in keep]))
    return dict(zip(keep, q))


@pytest.mark.parametrize("t,k,p", [(0.7, 5, 0.9), (1.0, 0, 1.0), (1.7, 3, 0.5), (0.3, 0, 0.99)])
def test_draw_frequencies_equal_the_kept_distribution(t, k, p):
    x = RNG.standard_normal(9) * 1.5
    expect = _brute_force_probs(list(x), t, k, p)
    n = 20000
    counts = {}
    for i in range(n):
        tok = sample(x, t, k, p, (i + 0.5) / n)
        counts[tok] = counts.get(tok, 0) + 1
    assert set(counts) <= set(expect)
    for tok, pr in expect.items():
        assert abs(counts.get(tok, 0) / n - pr) <= 1.0 / n + 1e-12


def test_sample_contract():
    assert contract.sample(logits=False, len_logits=4, rows=1, n=4, len_u=1) == contract.INVALID
    assert contract.sample(len_logits=0, rows=0, n=4, len_u=0) == contract.EMPTY
    assert contract.sample(len_logits=3, rows=1, n=4, len_u=1) == contract.LOGITS_LEN
    assert contract.sample(len_logits=4, rows=1, n=4, len_u=2) == contract.B_LEN
    assert contract.sample(len_logits=4, rows=1, n=4, len_u=1, temperature=-1.0) == contract.INVALID
    assert contract.sample(len_logits=4, rows=1, n=4, len_u=1, temperature=float("nan")) == contract.INVALID
    assert contract.sample(len_logits=4, rows=1, n=4, len_u=1, top_p=0.0) == contract.INVALID
    assert contract.sample(len_logits=4, rows=1, n=4, len_u=1, top_p=1.5) == contract.INVALID
    v = 128256
    assert contract.sample(len_logits=v, rows=1, n=v, len_u=1, top_k=50, top_p=0.95) == contract.OK
    assert contract.sample(len_logits=v, rows=1, n=v, len_u=1, top_k=0) == contract.TOO_LARGE
    assert contract.sample(len_logits=v, rows=1, n=v, len_u=1, top_k=0, temperature=0.0) == contract.OK
    assert contract.sample(len_logits=v, rows=1, n=v, len_u=1, top_k=1024) == contract.OK
    assert contract.sample(len_logits=v, rows=1, n=v, len_u=1, top_k=1025) == contract.TOO_LARGE
