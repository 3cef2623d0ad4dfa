"""Pins of the oracle's int8 K/V cache format (oracle.c: orc_q8_row; oracle/chunk.py: quantize_kv), on the CPU.

The pages name int8 K/V caches without fixing a format ("decode-ops", its opening paragraph; "Inside the
engine", "1. CausalLM"), so the format is the library's own: per (position, K/V head) row, s = max|x| / 127 in
fp32, codes rint(x / s) in fp32 with ties to even, clamped to [-127, 127]; the row stands for q * s.

  - a worked example with a scale that is a power of two (every division exact, so the codes are decided by
    hand, three of them on a tie);
  - special rows (zeros, one non-zero element, a negative maximum), the error bound |x - q s| <= s / 2 and the
    exact behaviour under scaling by powers of two, over seeded rows;
  - the chunked form's vectorised quantizer against the C one, bit for bit;
  - the decode step through an int8 cache: the token-by-token oracle and the chunked oracle (two independent
    forms of the same definition) agree on logits, hidden states and every stored code and scale, and the
    cache holds q8 of a position's K/V row at that position (the layout: codes, then scales).
"""
import ctypes

import numpy as np

import oracle
import synth
from oracle import chunk


def test_worked_example_power_of_two_scale():
    # max |x| = 7.9375 = 127 / 16, so s = 1/16 exactly and every code is 16 x, rounded half to even
    x = np.array([7.9375, -1.5, 0.03125, 0.09375, 0.15625, -0.15625, 3.0, -7.9375])
    q, s = oracle.q8_row(x)
    assert s == np.float32(0.0625)
    assert q.tolist() == [127, -24, 0, 2, 2, -2, 48, -127]   # 0.5 -> 0, 1.5 -> 2, 2.5 -> 2, -2.5 -> -2


def test_special_rows():
    q, s = oracle.q8_row(np.zeros(8))
    assert s == 0 and not q.any()
    q, s = oracle.q8_row(np.array([0.0, 0.0, -3.5, 0.0]))
    assert q.tolist() == [0, 0, -127, 0] and s == np.float32(np.float32(3.5) / np.float32(127))
    q, s = oracle.q8_row(np.array([-10.0, 4.0, 5.0]))          # the maximum magnitude is negative
    assert q[0] == -127 and s == np.float32(np.float32(10.0) / np.float32(127))


def test_bound_and_scaling_over_seeded_rows():
    rows = synth.normal((300, 128), 7, 1, 1.0).astype(np.float64)
    rows[5] *= 1e-30
    rows[9] *= 1e30
    for x in rows:
        q, s = oracle.q8_row(x)
        x32 = x.astype(np.float32).astype(np.float64)
        assert np.abs(q).max() == 127 and np.abs(q.astype(np.int32)).max() <= 127
        err = np.abs(x32 - q.astype(np.float64) * np.float64(s))
        assert err.max() <= np.float64(s) * (0.5 + 1e-6), err.max() / s
        for k in (-3, 4):                                    # scaling by 2^k scales s and keeps the codes
            q2, s2 = oracle.q8_row(x * 2.0 ** k)
            if np.isfinite(s2) and s2 > 0 and np.float32(s) * np.float32(2.0 ** k) > 1e-37:
                assert np.array_equal(q2, q) and s2 == np.float32(s * np.float32(2.0 ** k))


def test_chunk_quantizer_equals_c():
    rows = synth.normal((64, 3, 32), 8, 2, 2.0).astype(np.float64)
    rows[0, 1] = 0.0
    codes, scales = chunk.quantize_kv(rows)
    for r in range(64):
        for g in range(3):
            q, s = oracle.q8_row(rows[r, g])
            assert np.array_equal(codes[r, g], q) and scales[r, g] == s


def test_decode_through_int8_cache_token_and_chunk_forms_agree():
    s = synth.TINY.with_(kv_dtype="q8", head_dim=8, d=32, hidden=48)
    W = synth.model(s, seed=6)
    m = oracle.Model(s, W)
    toks = synth.prompt(12, s.vocab, stream=61).tolist()
    c1 = m.new_cache(16)
    lg1, hd1 = [], []
    for p, t in enumerate(toks):
        lg, hd = m.forward_token(t, p, c1, want_hidden=True)
        lg1.append(lg)
        hd1.append(hd)
    c2 = m.new_cache(16)
    lg2, hd2 = chunk.forward_chunk(s, chunk.Weights(s, W), toks, 0, c2)
    assert np.max(np.abs(np.array(lg1) - lg2)) <= 1e-9 * np.max(np.abs(lg2))
    assert np.max(np.abs(np.array(hd1) - hd2)) <= 1e-9 * np.max(np.abs(hd2))
    for l in range(s.n_layer):
        for w in ("k", "v"):
            assert np.array_equal(c1.codes(l, w)[:12], c2.codes(l, w)[:12])
            assert np.array_equal(c1.scales(l, w)[:12], c2.scales(l, w)[:12])
            assert not c1.codes(l, w)[12:].any() and not c1.scales(l, w)[12:].any()
    # layer 0 at position 0 sees only its own token: its K/V rows are q8 of the rows an fp64 cache stores
    k64 = [np.zeros((16, s.n_kv, s.head_dim)) for _ in range(s.n_layer)]
    v64 = [np.zeros((16, s.n_kv, s.head_dim)) for _ in range(s.n_layer)]
    c64 = oracle.Cache(s.with_(kv_dtype="f32"), 16)
    c64._kp = (ctypes.c_void_p * s.n_layer)(*[a.ctypes.data for a in k64])
    c64._vp = (ctypes.c_void_p * s.n_layer)(*[a.ctypes.data for a in v64])
    c64._c = oracle._Cache(c64._kp, c64._vp, 16)
    oracle.Model(s.with_(kv_dtype="f64"), W).forward_token(toks[0], 0, c64)
    for g in range(s.n_kv):
        for w, ref in (("k", k64[0]), ("v", v64[0])):
            q, sc = oracle.q8_row(ref[0, g])
            assert np.array_equal(c1.codes(0, w)[0, g], q) and c1.scales(0, w)[0, g] == sc
