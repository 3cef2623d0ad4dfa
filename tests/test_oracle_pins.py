"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test ties one oracle function to something other than itself: a value a page prints,
a closed form, an invariant, a special case that reduces to a textbook or library routine,
or brute force on a tiny input. The oracle is then trusted as the GPU path's reference.
"""
import math

import numpy as np
import pytest
import scipy.special

import oracle
import synth
from oracle import contract
from tests.conftest import golden

RNG = np.random.default_rng(1234)


def bf16_bits(values):
    """bf16 bit patterns of values that are exactly representable in bf16 (checked)."""
    f = np.asarray(values, dtype=np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((bits.astype(np.uint32) << 16).view(np.float32), f), "not bf16-exact"
    return bits


# ---------------------------------------------------------------------------------------------
# gemv_t and the head mat-vec
# ---------------------------------------------------------------------------------------------

def test_gemv_t_worked_example():
    g = golden("gemv_worked_example.json")
    a = np.array(g["a"], dtype=np.float32).reshape(g["m"], g["n"])
    y = oracle.gemv_t(a, np.array(g["x"]))
    assert y.tolist() == g["y"]
    assert contract.gemv_t(len_a=6, m=2, n=3, len_x=2, len_y=3) == g["status"]


def test_gemv_t_one_hot_returns_row_exactly():
    a = RNG.standard_normal((37, 53)).astype(np.float32)
    for i in (0, 17, 36):
        x = np.zeros(37)
        x[i] = 1.0
        assert np.array_equal(oracle.gemv_t(a, x), a[i].astype(np.float64))


@pytest.mark.parametrize("m,n", [(300, 300), (128, 1536)])
def test_gemv_t_against_library_sum(m, n):
    # the llmk page checks these two shapes to 1e-9 worst absolute delta against an independent kernel
    a = RNG.standard_normal((m, n))
    x = RNG.standard_normal(m)
    y = oracle.gemv_t(a, x)
    assert np.max(np.abs(y - a.T @ x)) <= 1e-9


def test_gemv_t_nonuniform_negative_weights_exact():
    # small integers: every partial sum is exact in fp64, so any order gives the same answer
    a = RNG.integers(-9, 10, size=(23, 31)).astype(np.float32)
    x = RNG.integers(-5, 6, size=23).astype(np.float64)
    y = oracle.gemv_t(a, x)
    ref = [sum(float(a[i, j]) * x[i] for i in range(23)) for j in range(31)]
    assert y.tolist() == ref


def test_gemv_t_reads_bf16_bits():
    vals = np.array([[1.5, -2.0, 0.15625], [3.0, 0.0078125, -1.0]], dtype=np.float32)
    y = oracle.gemv_t(bf16_bits(vals), np.array([2.0, -1.0]))
    assert y.tolist() == [0.0, -4.0078125, 1.3125]


def test_gemv_t_is_not_transposed_matvec():
    # a transposed operand would swap the roles; a non-square case catches it
    a = np.arange(6, dtype=np.float32).reshape(2, 3)
    assert oracle.gemv_t(a, np.array([1.0, 0.0])).tolist() == [0.0, 1.0, 2.0]
    assert oracle.matvec(a, np.array([1.0, 0.0, 0.0])).tolist() == [0.0, 3.0]


def test_matvec_equals_gemv_t_of_transpose_exactly():
    w = RNG.standard_normal((41, 29))
    x = RNG.standard_normal(29)
    assert np.array_equal(oracle.matvec(w, x), oracle.gemv_t(np.ascontiguousarray(w.T), x))


# ---------------------------------------------------------------------------------------------
# contract
# ---------------------------------------------------------------------------------------------

def test_contract_examples():
    g = golden("contract_examples.json")
    for case in g["residual_dims_check"]:
        assert contract.residual_dims_check(*case["args"]) == case["status"]
    for code, name in g["status_table"].items():
        assert contract.status_name(int(code)) == name
    fallback = contract.status_name(g["fallback_name_code"])
    for bad in (0, 559, 580, -1, 1 << 40):
        assert contract.status_name(bad) == fallback
    assert contract.MAX_DIM == g["max_dim"]


def test_contract_refusals():
    assert contract.residual_dims_check(0, 0, 0) == 561
    assert contract.residual_dims_check(-3, -3, -3) == 561
    assert contract.residual_dims_check((1 << 24) + 1, 0, 0) == 564
    assert contract.residual_dims_check(6, 6, 5) == 563
    assert contract.kv_append_dims_check(0, 0, 3, 3) == 560       # growth from an empty cache
    assert contract.kv_append_dims_check(6, 6, 0, 0) == 561       # an empty append is refused
    assert contract.kv_append_dims_check(6, 5, 3, 3) == 566
    assert contract.kv_append_dims_check(6, 6, 3, 2) == 567
    assert contract.argmax_dims_check(0, 0) == 561
    assert contract.argmax_dims_check(4, 3) == 568
    assert contract.gemv_dims_check(2, 3, 5, 2) == 569
    assert contract.gemv_dims_check(2, 3, 6, 3) == 570
    assert contract.gemv_dims_check(0, 3, 0, 0) == 561
    assert contract.kv_append_flat(capacity=8, cache_len=6, len_cache=6, n_new=3, len_new=3) == 571
    # the same append into slot 1 of a pool whose slots hold 4 positions of 2 x 2 elements (plane 16): the
    # page's cache of 6 grows to 9, written at the slot's base plus the old fill
    pool = dict(n_layer=1, n_slots=2, capacity=4, n_kv=2, head_dim=2)
    assert contract.kv_append(pool, 0, 1, 0, 6, 6, True, 3, 3) == (560, 9, 16 + 6)
    assert contract.kv_append(pool, 0, 1, 1, 6, 5, True, 3, 3)[0] == 566
    assert contract.kv_append(pool, 0, 1, 0, 14, 14, True, 3, 3)[0] == 571
    assert contract.kv_append(pool, 0, 2, 0, 6, 6, True, 3, 3)[0] == 575


# ---------------------------------------------------------------------------------------------
# K/V append
# ---------------------------------------------------------------------------------------------

def test_kv_append_worked_example():
    g = golden("kv_append_example.json")
    out = oracle.kv_append_copy(np.array(g["cache"]), np.array(g["new_vals"]))
    assert out.tolist() == g["out"] and out.size == g["n"]


def test_kv_append_growth_from_empty_and_order():
    out = oracle.kv_append_copy(np.zeros(0, np.float32), np.array([7.0, 8.0]))
    out = oracle.kv_append_copy(out, np.array([9.0]))
    assert out.tolist() == [7.0, 8.0, 9.0]


def test_kv_append_bf16_rounds_to_nearest_even():
    vals = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -9, -(1.0 + 3 * 2.0 ** -8), 3.0e38, np.nan],
                    dtype=np.float32)
    out = oracle.kv_append_copy(np.zeros(0, np.uint16), vals, dtype="bf16")
    back = oracle.bf16_to_f64(out)
    assert back[0] == 1.0                 # tie -> even mantissa (down)
    assert back[1] == 1.0 + 4 * 2.0 ** -8  # tie -> even mantissa (up)
    assert back[2] == 1.0                 # below half -> down
    assert back[3] == -(1.0 + 4 * 2.0 ** -8)
    assert back[4] > 3.0e38 and math.isfinite(back[4])
    assert math.isnan(back[5])


# ---------------------------------------------------------------------------------------------
# argmax
# ---------------------------------------------------------------------------------------------

def test_argmax_examples():
    g = golden("argmax_examples.json")
    for case in g["cases"]:
        tok, val = oracle.argmax(np.array(case["logits"], dtype=np.float32))
        assert tok == case["token_id"]
        if "logit" in case:
            assert val == case["logit"]
    n, at = g["wide_row"]["n"], g["wide_row"]["planted_max_at"]
    row = synth.normal((n,), 10, 0, 3.0)
    row[at] = row.max() + 1.0
    assert oracle.argmax(row)[0] == at


def test_argmax_brute_force_and_numpy():
    for trial in range(200):
        n = int(RNG.integers(1, 40))
        row = RNG.integers(-3, 4, size=n).astype(np.float32)   # many exact ties
        tok, val = oracle.argmax(row)
        first = min(i for i in range(n) if row[i] == row.max())
        assert tok == first == int(np.argmax(row)) and val == row.max()


def test_argmax_signed_zero_and_nan():
    assert oracle.argmax(np.array([-0.0, 0.0, -1.0], np.float32))[0] == 0
    assert oracle.argmax(np.array([0.0, -0.0], np.float32))[0] == 0
    row = np.array([1.0, np.nan, 5.0, np.nan], np.float32)
    assert oracle.argmax(row)[0] == 1 == int(np.argmax(row))
    assert oracle.argmax(np.array([-np.inf, -np.inf], np.float32))[0] == 0


# ---------------------------------------------------------------------------------------------
# residual add, RMSNorm, SiLU
# ---------------------------------------------------------------------------------------------

def test_residual_worked_example_and_wide():
    g = golden("residual_example.json")
    assert oracle.residual_add_f32(np.array(g["a"]), np.array(g["b"])).tolist() == g["out"]
    a = RNG.standard_normal(g["wide_n"]).astype(np.float32)
    b = RNG.standard_normal(g["wide_n"]).astype(np.float32)
    delta = np.abs(oracle.residual_add_f32(a, b).astype(np.float64) - (a + b).astype(np.float64))
    assert delta.max() == g["wide_max_abs_delta"]


def test_rmsnorm_closed_forms():
    h = oracle.rmsnorm(np.array([3.0, 4.0]), np.ones(2), 1e-5)
    assert np.allclose(h, np.array([3.0, 4.0]) / math.sqrt(12.5 + 1e-5), rtol=1e-15, atol=0)
    for c in (0.5, 2.0, -7.0):
        h = oracle.rmsnorm(np.full(64, c), np.ones(64), 1e-5)
        assert np.allclose(h, c / math.sqrt(c * c + 1e-5), rtol=1e-14, atol=0)
    x = RNG.standard_normal(4096)
    h = oracle.rmsnorm(x, np.ones(4096), 1e-5)
    ms = np.mean(x * x)
    assert abs(np.mean(h * h) - ms / (ms + 1e-5)) < 1e-12
    g = RNG.standard_normal(4096).astype(np.float32)
    assert np.allclose(oracle.rmsnorm(x, g, 1e-5), h * g.astype(np.float64), rtol=1e-14, atol=1e-300)


def test_add_rmsnorm_updates_residual_then_norms():
    r = RNG.standard_normal((3, 16)).astype(np.float32)
    x = RNG.standard_normal((3, 16)).astype(np.float32)
    g = np.ones(16, np.float32)
    r2, h = oracle.add_rmsnorm_f32(r, x, g, 3, 16, 1e-5)
    assert np.array_equal(r2, r + x)
    for row in range(3):
        ms = np.mean(r2[row].astype(np.float64) ** 2)
        assert np.allclose(h[row], r2[row] / np.sqrt(ms + 1e-5), rtol=1e-6)
    r3, h3 = oracle.add_rmsnorm_f32(r, None, g, 3, 16, 1e-5)
    assert np.array_equal(r3, r)


def test_silu_closed_form():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) / 40.0 - 1.0) < 1e-15
    assert abs(oracle.silu(-40.0)) < 1e-15
    for z in np.linspace(-8, 8, 33):
        assert abs(oracle.silu(z) - z * scipy.special.expit(z)) <= 1e-15 * max(1.0, abs(z))
    gate = RNG.standard_normal(100).astype(np.float32)
    up = RNG.standard_normal(100).astype(np.float32)
    out = oracle.silu_mul_f32(gate, up)
    ref = (gate.astype(np.float64) * scipy.special.expit(gate.astype(np.float64)) * up).astype(np.float32)
    assert np.array_equal(out, ref)


# ---------------------------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("layout", [oracle.HALF_SPLIT, oracle.INTERLEAVED])
def test_rope_identity_at_zero_and_norm_preserving(layout):
    v = RNG.standard_normal(3 * 8)
    assert np.array_equal(oracle.rope(v, 3, 8, 0, 1e4, layout), v)
    r = oracle.rope(v, 3, 8, 123, 1e4, layout)
    if layout == oracle.HALF_SPLIT:
        pairs = lambda u: [(u[h * 8 + j], u[h * 8 + j + 4]) for h in range(3) for j in range(4)]
    else:
        pairs = lambda u: [(u[h * 8 + 2 * j], u[h * 8 + 2 * j + 1]) for h in range(3) for j in range(4)]
    for (a, b), (c, d) in zip(pairs(v), pairs(r)):
        assert abs(math.hypot(a, b) - math.hypot(c, d)) < 1e-12


def test_rope_inverse_and_relative_position():
    q = RNG.standard_normal(16)
    k = RNG.standard_normal(16)
    back = oracle.rope(oracle.rope(q, 1, 16, 77, 1e4), 1, 16, -77, 1e4)
    assert np.allclose(back, q, atol=1e-12)
    dots = [np.dot(oracle.rope(q, 1, 16, p + 5, 1e4), oracle.rope(k, 1, 16, p, 1e4)) for p in (0, 9, 400)]
    assert max(dots) - min(dots) < 1e-11


def test_rope_hd2_is_plain_rotation_by_pos_radians():
    v = np.array([0.6, -0.8])
    for pos in (1, 2, 1000):
        c, s = math.cos(pos), math.sin(pos)
        expect = [0.6 * c + 0.8 * s, 0.6 * s - 0.8 * c]
        assert np.allclose(oracle.rope(v, 1, 2, pos, 1e6), expect, atol=1e-15)


def test_rope_layouts_are_a_permutation_of_each_other():
    # half-split pair (j, j+hd/2) of v is interleaved pair (2j, 2j+1) of the permuted vector
    hd = 8
    v = RNG.standard_normal(2 * hd)
    perm = [h * hd + (j // 2 if j % 2 == 0 else hd // 2 + j // 2) for h in range(2) for j in range(hd)]
    inter = oracle.rope(v[perm], 2, hd, 33, 1e4, oracle.INTERLEAVED)
    half = oracle.rope(v, 2, hd, 33, 1e4, oracle.HALF_SPLIT)
    assert np.allclose(inter, half[perm], atol=1e-14)


def test_rope_frequency_schedule():
    # pair j turns by pos * base^(-2j/hd): with a one-hot in pair j, the angle is recoverable
    hd, base, pos = 8, 1e4, 3
    for j in range(hd // 2):
        v = np.zeros(hd)
        v[j] = 1.0
        r = oracle.rope(v, 1, hd, pos, base)
        angle = math.atan2(r[j + hd // 2], r[j])
        expect = pos * base ** (-2 * j / hd)
        assert abs(math.remainder(angle - expect, 2 * math.pi)) < 1e-12


def test_rope_table_is_the_rotation_of_unit_vectors():
    # rotating the unit vector of pair j's first element gives (cos, sin) of that pair's angle,
    # so the table must hold exactly what the (separately pinned) rotation does, rounded to fp32
    hd, base = 8, 1e4
    t = oracle.rope_table_f32(50, hd, base).reshape(50, hd // 2, 2)
    for p in (0, 1, 17, 49):
        for j in range(hd // 2):
            e = np.zeros(hd)
            e[j] = 1.0
            r = oracle.rope(e, 1, hd, p, base, oracle.HALF_SPLIT)
            assert t[p, j, 0] == np.float32(r[j]) and t[p, j, 1] == np.float32(r[j + hd // 2])


# ---------------------------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------------------------

def test_attend_single_position_returns_v0():
    k = RNG.standard_normal((1, 2, 4)).astype(np.float32)
    v = RNG.standard_normal((1, 2, 4)).astype(np.float32)
    out = oracle.attend(RNG.standard_normal(16), k, v, 4, 2, 4)
    expect = np.concatenate([v[0, 0], v[0, 0], v[0, 1], v[0, 1]]).astype(np.float64)
    assert np.array_equal(out, expect)


def test_attend_equal_keys_gives_mean_of_values():
    k = np.repeat(RNG.standard_normal((1, 1, 8)), 9, axis=0).astype(np.float32)
    v = RNG.standard_normal((9, 1, 8)).astype(np.float32)
    out = oracle.attend(RNG.standard_normal(8), k, v, 1, 1, 8)
    assert np.allclose(out, v[:, 0].astype(np.float64).mean(axis=0), atol=1e-14)


def test_attend_group_mapping_and_softmax_library():
    ctx, H, Hkv, hd = 7, 6, 2, 4
    q = RNG.standard_normal(H * hd)
    k = RNG.standard_normal((ctx, Hkv, hd))
    v = RNG.standard_normal((ctx, Hkv, hd))
    out = oracle.attend(q, k, v, H, Hkv, hd).reshape(H, hd)
    for h in range(H):
        g = h // (H // Hkv)                    # heads 0,1,2 -> K/V head 0; 3,4,5 -> 1
        w = scipy.special.softmax(k[:, g] @ q[h * hd:(h + 1) * hd] / 2.0)
        assert np.allclose(out[h], w @ v[:, g], atol=1e-13)


def test_attend_mha_special_case():
    ctx, H, hd = 5, 3, 4
    q = RNG.standard_normal(H * hd)
    k = RNG.standard_normal((ctx, H, hd))
    v = RNG.standard_normal((ctx, H, hd))
    out = oracle.attend(q, k, v, H, H, hd).reshape(H, hd)
    for h in range(H):
        w = scipy.special.softmax(k[:, h] @ q[h * hd:(h + 1) * hd] / 2.0)
        assert np.allclose(out[h], w @ v[:, h], atol=1e-13)


# ---------------------------------------------------------------------------------------------
# the whole step: the Inference Academy page's printed run
# ---------------------------------------------------------------------------------------------

def _page_model(n_kv=None, layout=oracle.INTERLEAVED):
    g = golden("page_decode.json")["config"]
    s = synth.TINY.with_(rope_layout=layout)
    if n_kv is not None:
        s = s.with_(n_kv=n_kv)
    assert (s.vocab, s.d, s.n_layer, s.n_head, s.hidden, s.max_seq, s.head_dim) == \
        (g["vocab"], g["d"], g["n_layer"], g["n_head"], g["hidden"], g["max_seq"], g["head_dim"])
    return s, oracle.Model(s, synth.page_draws(s, seed=g["seed"], std=g["weight_std"]))


def test_page_run_reproduces_printed_tokens():
    g = golden("page_decode.json")
    s, m = _page_model()
    toks, _, _ = oracle.generate(m, g["prompt"], g["n_new"], s.max_seq)
    assert toks[:3] == g["printed_first_tokens"]
    assert (oracle.recompute_generate(m, g["prompt"], g["n_new"], s.max_seq) == toks) == g["printed_cache_equals_recompute"]


@pytest.mark.parametrize("layout", [oracle.HALF_SPLIT, oracle.INTERLEAVED])
@pytest.mark.parametrize("n_kv", [2, 4, 1])
def test_cache_equals_recompute(layout, n_kv):
    g = golden("page_decode.json")
    s, m = _page_model(n_kv=n_kv, layout=layout)
    toks, _, _ = oracle.generate(m, g["prompt"], g["n_new"], s.max_seq)
    assert oracle.recompute_generate(m, g["prompt"], g["n_new"], s.max_seq) == toks


def test_kv_bytes_per_token():
    g = golden("page_decode.json")
    s = synth.TINY
    cache = oracle.Cache(s.with_(kv_dtype="f32"), 1)
    elems_per_token = sum(a[0].size for a in cache.k) + sum(a[0].size for a in cache.v)
    assert elems_per_token * 2 == g["kv_bytes_per_token_fp16"]
    mha = oracle.Cache(s.with_(n_kv=g["exercise_full_mha_n_kv"]), 1)
    assert (sum(a[0].size for a in mha.k) + sum(a[0].size for a in mha.v)) * 2 == g["kv_bytes_per_token_fp16_full_mha"]


def test_logits_follow_final_hidden_state():
    # logits = out . rmsnorm(x_L): recomputing the head from the returned hidden state agrees to fp32 rounding
    s, m = _page_model()
    c = m.new_cache(s.max_seq)
    for pos, t in enumerate((3, 14, 15)):
        logits, hidden = m.forward_token(t, pos, c, want_hidden=True)
    W = m.W
    ref = oracle.matvec(W["out"], oracle.rmsnorm(hidden[-1].astype(np.float64), W["norm"], s.eps))
    assert np.max(np.abs(logits - ref)) < 1e-5


def test_forward_token_refuses_out_of_range():
    s, m = _page_model()
    c = m.new_cache(8)
    with pytest.raises(ValueError):
        m.forward_token(40, 0, c)
    with pytest.raises(ValueError):
        m.forward_token(1, 8, c)


# ---------------------------------------------------------------------------------------------
# the chunked forward (oracle/chunk.py): the same step for many rows at once, held to the
# token-by-token oracle (itself pinned above) and to the page's printed tokens
# ---------------------------------------------------------------------------------------------

from oracle import chunk  # noqa: E402

MID = synth.Shape("mid bf16 (V300 d64 L2 H4/2 hd16 F96)", 300, 64, 2, 4, 2, 16, 96, 96, 1e-5, 1e4,
                  synth.ROPE_HALF_SPLIT, "bf16", "bf16", 0.08)


def _close(a, b, tol=1e-9):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)) <= tol


def _bf16_ulps(a, b):
    """Largest distance in bf16 steps between two arrays of bf16 bit patterns of the same sign pattern."""
    return int(np.max(np.abs(a.astype(np.int64) - b.astype(np.int64)))) if a.size else 0


@pytest.mark.parametrize("shape_name,layout", [("tiny", synth.ROPE_INTERLEAVED), ("tiny", synth.ROPE_HALF_SPLIT),
                                               ("mid", synth.ROPE_HALF_SPLIT), ("mid", synth.ROPE_INTERLEAVED)])
def test_chunk_forward_equals_token_by_token(shape_name, layout):
    """A prompt as two chunks (10 rows, then 30) gives the token-by-token oracle's logits, hidden states and
    K/V (fp64 sums in another order: relative 1e-9; stored K/V at most one step of their dtype apart)."""
    if shape_name == "tiny":
        s = synth.TINY.with_(rope_layout=layout)
        W = synth.as_f32(synth.page_draws(s))
    else:
        s = MID.with_(rope_layout=layout)
        W = synth.model(s, seed=5)
    toks = synth.prompt(40, s.vocab, stream=50).tolist()
    m = oracle.Model(s, W)
    c1 = m.new_cache(s.max_seq)
    ref = [m.forward_token(t, p, c1, want_hidden=True) for p, t in enumerate(toks)]
    c2 = m.new_cache(s.max_seq)
    w = chunk.Weights(s, W)
    lg_a, hid_a = chunk.forward_chunk(s, w, toks[:10], 0, c2)
    lg_b, hid_b = chunk.forward_chunk(s, w, toks[10:], 10, c2)
    lg, hid = np.concatenate([lg_a, lg_b]), np.concatenate([hid_a, hid_b])
    for p in range(len(toks)):
        assert _close(lg[p], ref[p][0]) and _close(hid[p], ref[p][1]), p
        assert oracle.argmax(lg[p])[0] == oracle.argmax(ref[p][0])[0]
    for l in range(s.n_layer):
        for a, b in ((c1.k[l], c2.k[l]), (c1.v[l], c2.v[l])):
            if s.kv_dtype == "bf16":
                assert _bf16_ulps(a[:40], b[:40]) <= 1
            else:
                assert _close(a[:40], b[:40], 1e-6)


def test_chunk_forward_reproduces_the_pages_printed_tokens():
    """The page's prompt through one chunk, then one-row chunks fed their own greedy tokens: the page's
    printed first tokens, and the token-by-token oracle's whole run."""
    g = golden("page_decode.json")
    s = synth.TINY.with_(rope_layout=synth.ROPE_INTERLEAVED)
    W = synth.as_f32(synth.page_draws(s, seed=g["config"]["seed"], std=g["config"]["weight_std"]))
    m = oracle.Model(s, W)
    ref, _, _ = oracle.generate(m, g["prompt"], g["n_new"], s.max_seq)
    w = chunk.Weights(s, W)
    c = m.new_cache(s.max_seq)
    lg, _ = chunk.forward_chunk(s, w, g["prompt"], 0, c, want_hidden=False)
    toks = [oracle.argmax(lg[-1])[0]]
    pos = len(g["prompt"])
    while len(toks) < g["n_new"]:
        lg, _ = chunk.forward_chunk(s, w, [toks[-1]], pos, c, want_hidden=False)
        toks.append(oracle.argmax(lg[0])[0])
        pos += 1
    assert toks[:3] == g["printed_first_tokens"]
    assert toks == ref


def test_forward_rows_equals_each_sequence_stepped_alone():
    """Five sequences at ragged lengths, one batched step: each row's logits, hidden state and appended K/V
    equal that sequence's token-by-token step."""
    s = MID
    W = synth.model(s, seed=6)
    m = oracle.Model(s, W)
    lens = [1, 7, 30, 2, 55]
    caches, toks = [], []
    for b, n in enumerate(lens):
        c = m.new_cache(s.max_seq)
        for p, t in enumerate(synth.prompt(n, s.vocab, stream=60 + b).tolist()):
            m.forward_token(t, p, c)
        caches.append(c)
        toks.append(int(synth.prompt(1, s.vocab, stream=70 + b)[0]))
    pre = [(np.array([c.k[l][:n].copy() for l in range(s.n_layer)]), np.array([c.v[l][:n].copy() for l in range(s.n_layer)]))
           for c, n in zip(caches, lens)]
    w = chunk.Weights(s, W)
    def prefix(l, b):   # the cached positions in two head-major pieces (the split of a context is immaterial)
        k, v, h = pre[b][0][l].transpose(1, 0, 2), pre[b][1][l].transpose(1, 0, 2), lens[b] // 2
        return [(k[:, :h], v[:, :h]), (k[:, h:], v[:, h:])]

    lg, hid, new_kv = chunk.forward_rows(s, w, toks, lens, prefix)
    for b, (c, n) in enumerate(zip(caches, lens)):
        ref_lg, ref_hid = m.forward_token(toks[b], n, c, want_hidden=True)
        assert _close(lg[b], ref_lg) and _close(hid[b], ref_hid), b
        for l in range(s.n_layer):
            assert _bf16_ulps(new_kv[l][0][b], c.k[l][n]) <= 1 and _bf16_ulps(new_kv[l][1][b], c.v[l][n]) <= 1


def test_round_kv_matches_the_c_oracle_rounding():
    vals = np.concatenate([np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 3 * 2.0 ** -8), np.nan, 3.0e38,
                                     -np.inf, 0.0, -0.0]), synth.normal((2000,), 71, 0, 3.0).astype(np.float64)])
    assert np.array_equal(chunk.round_kv(vals, "bf16"), oracle.f32_to_bf16(vals.astype(np.float32)))
    assert np.array_equal(chunk.to_f64(chunk.round_kv(vals, "bf16")[8:]),
                          oracle.bf16_to_f64(oracle.f32_to_bf16(vals[8:].astype(np.float32))))
