"""Pins of the oracle's int8 weight packs (oracle/quant.py) against what the format's definition fixes by
itself: values on the code grid come back exactly, the largest magnitude of a group takes code +-127, the
reconstruction error is at most half a step (plus one fp32 rounding of the quotient), ties round to even,
all-zero groups, exact power-of-two scaling, the byte layout of a pack built by hand, the grouping axis of a
model's projections, and the fp64-weight path of the C oracle reproducing its pinned fp32-weight path."""
import struct

import numpy as np
import pytest

import oracle
import synth
from oracle import quant

G = quant.GROUP


def grid_rows(rng, rows, K):
    """Rows whose every group holds k * 2^-e (integers |k| <= 127, one of them +-127): on the code grid."""
    k = rng.integers(-127, 128, size=(rows, K // G, G))
    k[..., 0] = np.where(rng.random((rows, K // G)) < 0.5, 127, -127)
    e = rng.integers(-12, 4, size=(rows, K // G, 1))
    return (k * np.exp2(e.astype(np.float64))).reshape(rows, K).astype(np.float32), k.reshape(rows, K)


def test_grid_values_round_trip_exactly():
    rng = np.random.default_rng(1)
    w, k = grid_rows(rng, 5, 3 * G)
    q, s = quant.quantize(w)
    assert np.array_equal(q.astype(np.int64), k)
    assert np.array_equal(quant.dequantize(q, s), w.astype(np.float64))
    # on the grid every q * s is exact in fp32 too, so the fp32 form of the weights agrees bit for bit
    assert np.array_equal(quant.dequantize(q, s, np.float32), w)


def test_error_within_half_a_step():
    rng = np.random.default_rng(2)
    for w in (rng.standard_normal((7, 4 * G)), rng.standard_t(2, (7, 4 * G)), rng.random((7, 4 * G)) * 1e-30):
        w = w.astype(np.float32)
        q, s = quant.quantize(w)
        err = np.abs(quant.dequantize(q, s) - w.astype(np.float64)).reshape(7, 4, G)
        # |w/s - rint(fl(w/s))| <= 1/2 + 127 * 2^-24 (one fp32 rounding of the quotient)
        assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 128 * 2.0 ** -24))


def test_largest_magnitude_takes_code_127():
    rng = np.random.default_rng(3)
    w = rng.standard_normal((4, 2 * G)).astype(np.float32)
    q, s = quant.quantize(w)
    g = w.reshape(4, 2, G)
    i = np.argmax(np.abs(g), axis=2)
    top = np.take_along_axis(q.reshape(4, 2, G), i[..., None], 2)[..., 0]
    sign = np.sign(np.take_along_axis(g, i[..., None], 2)[..., 0])
    assert np.array_equal(top, (127 * sign).astype(np.int8))
    assert np.all(np.abs(q.astype(np.int64)) <= 127)


def test_hand_group_rounds_half_to_even():
    # max |w| = 127 gives s = 1 exactly, so the codes are rint(w): ties go to the even neighbour
    w = np.zeros((1, G), np.float32)
    w[0, :8] = [127.0, -2.5, 3.5, 0.49, -0.5, 1.5, -126.51, 0.5]
    q, s = quant.quantize(w)
    assert s[0, 0] == 1.0
    assert q[0, :8].tolist() == [127, -2, 4, 0, 0, 2, -127, 0]
    assert not q[0, 8:].any()


def test_zero_group_and_scaling():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((3, 3 * G)).astype(np.float32)
    w[1, G:2 * G] = 0.0
    q, s = quant.quantize(w)
    assert s[1, 1] == 0.0 and not q[1, G:2 * G].any()
    assert np.all(s[s != 0] > 0)
    for e in (-20, 7):
        q2, s2 = quant.quantize(w * np.float32(2.0 ** e))
        assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(2.0 ** e))


def test_pack_layout_by_hand():
    rows, K = 2, 2 * G
    rng = np.random.default_rng(5)
    w = rng.standard_normal((rows, K)).astype(np.float32)
    q, s = quant.quantize(w)
    buf = quant.to_pack(q, s)
    assert buf.size == quant.pack_bytes(rows, K) == rows * K + 4 * rows * (K // G)
    hand = bytes(int(v) & 0xFF for v in q.ravel()) + b"".join(
        struct.pack("<f", float(s[r, g])) for r in range(rows) for g in range(K // G))
    assert buf.tobytes() == hand
    q2, s2 = quant.from_pack(buf, rows, K)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_model_projections_group_along_their_input():
    # a projection given [in][out] whose every output row is on the grid along `in` comes back exactly;
    # grouping along `out` instead would not (those groups are not on one grid)
    s0 = synth.TINY.with_(d=128, n_head=2, n_kv=1, head_dim=64, hidden=256, vocab=40)
    rng = np.random.default_rng(6)
    W = synth.model(s0, seed=0)
    for L in W["layers"]:
        for k in ("wq", "wk", "wv", "wo", "gate", "up", "down"):
            n_in, n_out = L[k].shape
            L[k] = np.ascontiguousarray(grid_rows(rng, n_out, n_in)[0].T)
    W["out"] = grid_rows(rng, s0.vocab, s0.d)[0]
    Q = quant.quantized_weights(W)
    Q32 = quant.quantized_weights(W, f64=False)
    assert all(np.array_equal(M[k], M32[k].astype(np.float64)) for M, M32 in zip(Q["layers"], Q32["layers"])
               for k in ("wq", "wk", "wv", "wo", "gate", "up", "down"))
    for L, M in zip(W["layers"], Q["layers"]):
        for k in ("wq", "wk", "wv", "wo", "gate", "up", "down"):
            assert np.array_equal(M[k], L[k].astype(np.float64)), k
    assert np.array_equal(Q["out"], W["out"].astype(np.float64))


def test_f64_weights_reproduce_the_f32_path():
    # the q8 reference model runs the oracle with fp64 weights; on weights exact in fp32 that path must give
    # bit-identical logits to the (pinned) fp32-weight path
    s0 = synth.TINY
    W = synth.model(s0, seed=3)
    W64 = {"emb": W["emb"].astype(np.float64), "out": W["out"].astype(np.float64), "norm": W["norm"],
           "layers": [{k: (v.astype(np.float64) if k not in ("n1", "n2") else v) for k, v in L.items()}
                      for L in W["layers"]]}
    a, b = oracle.Model(s0, W), oracle.Model(s0, W64)
    ca, cb = a.new_cache(8), b.new_cache(8)
    for pos, tok in enumerate([3, 17, 5, 29]):
        la, _ = a.forward_token(tok, pos, ca)
        lb, _ = b.forward_token(tok, pos, cb)
        assert np.array_equal(la, lb)


def test_quantize_refuses_ragged_groups():
    with pytest.raises(ValueError):
        quant.quantize(np.ones((2, G + 1), np.float32))
