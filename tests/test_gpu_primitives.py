"""Each primitive of the C ABI on the GPU against the oracle, element by element (MI355X only).

Sizes span several tiles and ragged tails, and include the primitive microbenchmark's full shapes:
gemv_t 4096x4096 bf16, add_rmsnorm 1x4096, RoPE on 32 q + 8 k heads at hd 128 for positions
0..8191, argmax over 128,256 logits N(0, 3) with planted exact ties.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from oracle import contract
from tests.conftest import golden
from tests.gpu_util import TOL, dev, host, rel_err, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sync():
    torch.cuda.synchronize()


def run_gemv_t(a_np, x_np):
    m, n = a_np.shape
    a = dev(a_np)
    x = dev(x_np.astype(np.float32))
    y = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.gemv_t_workspace_bytes(m, n, llmk.BF16 if a_np.dtype == np.uint16 else llmk.F32))
    st = llmk.gemv_t(a, x, y, m, n, ws)
    assert st == llmk.OK, llmk.status_name(st)
    _sync()
    return host(y)


# ---------------------------------------------------------------------------------------------
# gemv_t
# ---------------------------------------------------------------------------------------------

def test_gemv_t_worked_example():
    g = golden("gemv_worked_example.json")
    a = np.array(g["a"], dtype=np.float32).reshape(g["m"], g["n"])
    y = run_gemv_t(a, np.array(g["x"], np.float32))
    assert y.tolist() == g["y"]
    abf = (a.view(np.uint32) >> 16).astype(np.uint16)      # these values are exact in bf16
    assert run_gemv_t(abf, np.array(g["x"], np.float32)).tolist() == g["y"]


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("m,n", [(1, 8), (37, 53), (300, 300), (128, 1536), (1000, 4104), (4096, 6144),
                                 (14336, 4096), (4096, 28672)])
def test_gemv_t_matches_oracle(m, n, dt):
    say(f"gemv_t {m}x{n} {dt}")
    a = synth.normal((m, n), 11, m * 7 + n, 0.02, dt)
    x = synth.normal((m,), 12, m * 7 + n, 1.0)
    y = run_gemv_t(a, x)
    ref = oracle.gemv_t_f32(a, x)
    err = rel_err(y, ref)
    say(f"  rel err {err:.2e}")
    assert err <= TOL
    assert err <= 1e-4   # fp32 accumulation of these sizes stays far below the bar


def test_gemv_t_exact_on_integers_and_deterministic():
    # small integers: every partial sum is exact in fp32, so the result is exact in any order
    rng = np.random.default_rng(5)
    for m, n in [(1000, 4096), (333, 1000), (4096, 1024)]:
        a = rng.integers(-9, 10, size=(m, n)).astype(np.float32)
        x = rng.integers(-5, 6, size=m).astype(np.float32)
        y1 = run_gemv_t(a, x)
        assert np.array_equal(y1, oracle.gemv_t_f32(a, x))
        abf = (a.view(np.uint32) >> 16).astype(np.uint16)
        y2 = run_gemv_t(abf, x)
        assert np.array_equal(y2, y1)
    a = synth.normal((4096, 4096), 13, 0, 0.02, "bf16")
    x = synth.normal((4096,), 13, 1, 1.0)
    assert np.array_equal(run_gemv_t(a, x).view(np.uint32), run_gemv_t(a, x).view(np.uint32))


# ---------------------------------------------------------------------------------------------
# untransposed head mat-vec
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,dt", [(40, 16, "f32"), (1000, 1024, "bf16"), (777, 1001, "f32"),
                                          (151936, 1024, "bf16"), (128256, 4096, "bf16")])
def test_gemv_rowdot_matches_oracle(rows, cols, dt):
    say(f"gemv {rows}x{cols} {dt}")
    w = synth.normal((rows, cols), 14, rows + cols, 0.02, dt)
    x = synth.normal((cols,), 15, rows + cols, 1.0)
    y = torch.full((rows,), float("nan"), dtype=torch.float32, device="cuda")
    st = llmk.gemv(dev(w), dev(x), y, rows, cols)
    assert st == llmk.OK
    _sync()
    err = rel_err(host(y), oracle.matvec_f32(w, x))
    say(f"  rel err {err:.2e}")
    assert err <= TOL and err <= 1e-4


# ---------------------------------------------------------------------------------------------
# residual, add_rmsnorm, silu_mul
# ---------------------------------------------------------------------------------------------

def test_residual_add_worked_example_and_exact():
    g = golden("residual_example.json")
    a, b = dev(np.array(g["a"], np.float32)), dev(np.array(g["b"], np.float32))
    out = torch.empty(6, dtype=torch.float32, device="cuda")
    assert llmk.residual_add(a, b, out) == llmk.OK
    _sync()
    assert host(out).tolist() == g["out"]
    for n in (g["wide_n"], 100003):
        an, bn = synth.normal((n,), 16, n, 1.0), synth.normal((n,), 17, n, 1.0)
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        assert llmk.residual_add(dev(an), dev(bn), out) == llmk.OK
        _sync()
        assert np.max(np.abs(host(out).astype(np.float64) - oracle.residual_add_f32(an, bn))) == g["wide_max_abs_delta"]


@pytest.mark.parametrize("rows,n", [(1, 4096), (3, 1000), (5, 16), (2, 14336)])
@pytest.mark.parametrize("with_x", [True, False])
def test_add_rmsnorm_matches_oracle(rows, n, with_x):
    r = synth.normal((rows * n,), 18, n, 1.0)
    x = synth.normal((rows * n,), 19, n, 1.0) if with_x else None
    g = synth.normal((n,), 20, n, 0.1, mean=1.0)
    rd = dev(r)
    h = torch.empty(rows * n, dtype=torch.float32, device="cuda")
    st = llmk.add_rmsnorm(rd, None if x is None else dev(x), dev(g), h, rows, n, 1e-5)
    assert st == llmk.OK
    _sync()
    r_ref, h_ref = oracle.add_rmsnorm_f32(r, x, g, rows, n, 1e-5)
    assert np.array_equal(host(rd), r_ref)          # the residual update is one exactly rounded add
    assert rel_err(host(h), h_ref) <= TOL
    assert rel_err(host(h), h_ref) <= 1e-5


def test_silu_mul_matches_oracle():
    n = 14336 * 3 + 7
    gate = synth.normal((n,), 21, 0, 3.0)
    up = synth.normal((n,), 21, 1, 1.0)
    gate[:3] = [0.0, 80.0, -80.0]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    assert llmk.silu_mul(dev(gate), dev(up), out) == llmk.OK
    _sync()
    ref = oracle.silu_mul_f32(gate, up)
    got = host(out)
    assert got[0] == 0.0
    assert rel_err(got, ref) <= TOL and rel_err(got, ref) <= 1e-5


# ---------------------------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("base", [1e4, 5e5])
def test_rope_table_matches_oracle(base):
    max_pos, hd = 8192, 128
    t = torch.empty(max_pos * hd, dtype=torch.float32, device="cuda")
    assert llmk.rope_table_init(t, max_pos, hd, base) == llmk.OK
    _sync()
    ref = oracle.rope_table_f32(max_pos, hd, base)
    assert np.max(np.abs(host(t) - ref)) <= 2.0 ** -23   # both from fp64 angles; at most one fp32 ulp apart


@pytest.mark.parametrize("layout", [llmk.ROPE_HALF_SPLIT, llmk.ROPE_INTERLEAVED])
def test_rope_positions_0_to_8191(layout):
    rows, nq, nk, hd, base = 8192, 32, 8, 128, 1e4
    q = synth.normal((rows * nq * hd,), 22, 0, 1.0)
    k = synth.normal((rows * nk * hd,), 22, 1, 1.0)
    t = torch.empty(rows * hd, dtype=torch.float32, device="cuda")
    assert llmk.rope_table_init(t, rows, hd, base) == llmk.OK
    qd, kd = dev(q), dev(k)
    pos = torch.arange(rows, dtype=torch.int32, device="cuda")
    assert llmk.rope(qd, kd, rows, nq, nk, hd, pos, t, rows, layout) == llmk.OK
    _sync()
    q_ref, k_ref = oracle.rope_f32(q, k, rows, nq, nk, hd, 0, base, layout)
    eq, ek = rel_err(host(qd), q_ref), rel_err(host(kd), k_ref)
    say(f"rope layout {layout}: q err {eq:.2e} k err {ek:.2e}")
    assert eq <= TOL and ek <= TOL and eq <= 1e-5 and ek <= 1e-5


def test_rope_single_position_and_tiny_heads():
    for hd, pos0 in [(4, 5), (2, 63), (128, 4095)]:
        q = synth.normal((3 * hd,), 23, hd, 1.0)
        t = torch.empty(4096 * hd, dtype=torch.float32, device="cuda")
        assert llmk.rope_table_init(t, 4096, hd, 1e4) == llmk.OK
        qd = dev(q)
        pos = torch.tensor([pos0], dtype=torch.int32, device="cuda")
        assert llmk.rope(qd, None, 1, 3, 0, hd, pos, t, 4096, 0) == llmk.OK
        _sync()
        q_ref, _ = oracle.rope_f32(q, None, 1, 3, 0, hd, pos0, 1e4, 0)
        assert rel_err(host(qd), q_ref) <= 1e-5


@pytest.mark.parametrize("layout", [llmk.ROPE_HALF_SPLIT, llmk.ROPE_INTERLEAVED])
def test_rope_device_positions_per_row(layout):
    """Each row at its own device position (a batch of sequences at different lengths); rows whose
    position has no table row are left unchanged."""
    rows, nq, nk, hd, max_pos, base = 37, 4, 2, 64, 5000, 5e5
    positions = [int(p) for p in synth.ints((rows,), 0, max_pos - 1, 28, 0)]
    positions[3], positions[11], positions[20] = -1, max_pos, max_pos - 1
    q = synth.normal((rows * nq * hd,), 29, 0, 1.0)
    k = synth.normal((rows * nk * hd,), 29, 1, 1.0)
    t = torch.empty(max_pos * hd, dtype=torch.float32, device="cuda")
    assert llmk.rope_table_init(t, max_pos, hd, base) == llmk.OK
    qd, kd = dev(q), dev(k)
    pos = torch.tensor(positions, dtype=torch.int32, device="cuda")
    assert llmk.rope(qd, kd, rows, nq, nk, hd, pos, t, max_pos, layout) == llmk.OK
    _sync()
    gq, gk = host(qd).reshape(rows, -1), host(kd).reshape(rows, -1)
    qr, kr = q.reshape(rows, -1), k.reshape(rows, -1)
    for r, p in enumerate(positions):
        if 0 <= p < max_pos:
            q_ref, k_ref = oracle.rope_f32(qr[r], kr[r], 1, nq, nk, hd, p, base, layout)
            assert rel_err(gq[r], q_ref) <= 1e-5 and rel_err(gk[r], k_ref) <= 1e-5, (r, p)
        else:
            assert np.array_equal(gq[r], qr[r]) and np.array_equal(gk[r], kr[r]), (r, p)


# ---------------------------------------------------------------------------------------------
# K/V append
# ---------------------------------------------------------------------------------------------

def test_kv_append_worked_example_in_place():
    g = golden("kv_append_example.json")
    cache = torch.full((16,), -1.0, dtype=torch.float32, device="cuda")
    cache[:6] = torch.tensor(g["cache"], device="cuda")
    st, n = llmk.kv_append_flat(cache, g["cache_len"], g["cache_len"], dev(np.array(g["new_vals"], np.float32)))
    assert st == llmk.OK and n == g["n"]
    _sync()
    c = host(cache)
    assert c[:n].tolist() == g["out"]
    assert c[n:].tolist() == [-1.0] * (16 - n)        # nothing past the append is touched


def test_kv_append_bf16_rounding_matches_oracle():
    vals = np.concatenate([np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 3 * 2.0 ** -8), np.nan, 3.0e38],
                                    np.float32), synth.normal((4096,), 24, 0, 1.0)])
    cache = torch.zeros(8192, dtype=torch.bfloat16, device="cuda")
    st, n = llmk.kv_append_flat(cache, 0, 0, dev(vals))
    assert st == llmk.OK and n == vals.size
    _sync()
    ref = oracle.kv_append_copy(np.zeros(0, np.uint16), vals, "bf16")
    got = host(cache)[:n]
    assert np.array_equal(got, ref)
    st, n2 = llmk.kv_append_flat(cache, n, n, dev(vals[:3]))
    assert st == llmk.OK and n2 == n + 3
    st, _ = llmk.kv_append_flat(cache, n2, n2, dev(np.zeros(8192 - n2 + 1, np.float32)))
    assert st == 571


# ---------------------------------------------------------------------------------------------
# grouped-query attention
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("ctx,H,Hkv,hd,dt", [(1, 4, 2, 4, "f32"), (5, 4, 2, 4, "f32"), (16, 4, 4, 4, "f32"),
                                             (65, 8, 2, 64, "bf16"), (130, 32, 8, 128, "bf16"),
                                             (2100, 16, 8, 128, "f32"), (4352, 32, 8, 128, "bf16"),
                                             (8320, 32, 8, 128, "bf16"), (333, 6, 3, 2, "f32")])
def test_gqa_attend_matches_oracle(ctx, H, Hkv, hd, dt):
    say(f"attend ctx={ctx} H={H} Hkv={Hkv} hd={hd} {dt}")
    q = synth.normal((H * hd,), 25, ctx, 1.0)
    k = synth.normal((ctx, Hkv, hd), 26, ctx, 1.0, dt)
    v = synth.normal((ctx, Hkv, hd), 27, ctx, 1.0, dt)
    out = torch.full((H * hd,), float("nan"), dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.gqa_attend_workspace_bytes(ctx, H, hd))
    st = llmk.gqa_attend_flat(dev(q), dev(k), dev(v), ctx, H, Hkv, hd, out, ws)
    assert st == llmk.OK, llmk.status_name(st)
    _sync()
    ref = oracle.attend_f32(q, k, v, ctx, H, Hkv, hd)
    err = rel_err(host(out), ref)
    say(f"  rel err {err:.2e}")
    assert err <= TOL
    if ctx == 1:
        assert np.array_equal(host(out).reshape(H, hd),
                              np.repeat(oracle.bf16_to_f64(v[0]) if dt == "bf16" else v[0], H // Hkv, axis=0)
                              .astype(np.float32))


# ---------------------------------------------------------------------------------------------
# the pool-level append and attention: offsets, records and values against the oracle
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_pool_append_offsets_and_attend(dt):
    """Decode-style appends of one position (n_kv * hd elements) into (layer, slot) buffers of a pool:
    the offset each call returns equals the closed form bit-exactly, the written values are the oracle's
    rounding of the new values, nothing else changes, and attention over the slot equals the oracle's."""
    n_layer, n_slots, cap, Hkv, hd, H = 2, 3, 96, 2, 64, 8
    kv = llmk.BF16 if dt == "bf16" else llmk.F32
    pool = llmk.KVPool(n_layer, n_slots, cap, Hkv, hd, kv)
    row = Hkv * hd
    fields = dict(n_layer=n_layer, n_slots=n_slots, capacity=cap, n_kv=Hkv, head_dim=hd, dtype=kv)
    before = {(l, w): host(t).copy() for l in range(n_layer) for w, t in ((0, pool.k[l]), (1, pool.v[l]))}
    written = {}
    slot, layer, n_pos = 2, 1, 70
    vals = {w: synth.normal((n_pos, row), 30 + w, 0, 1.0) for w in (0, 1)}
    for p in range(n_pos):
        for w in (0, 1):
            cl = p * row
            exp = contract.kv_append(fields, layer, slot, w, cl, cl, True, row, row)
            st, nl, off = llmk.kv_append(pool, layer, slot, w, cl, dev(vals[w][p]))
            assert (st, nl, off) == exp, (p, w)
            st2, off2 = llmk.kv_slot_offset(pool, slot, p, 0)
            assert st2 == llmk.OK and off2 == off and contract.kv_slot_offset(n_slots, cap, Hkv, hd, slot, p, 0)[1] == off
    assert pool.len_k[layer, slot] == pool.len_v[layer, slot] == n_pos * row
    # a wrong claim of the fill is refused and changes nothing
    st, _, _ = llmk.kv_append(pool, layer, slot, 0, (n_pos - 1) * row, dev(vals[0][0]))
    assert st == 566 and pool.len_k[layer, slot] == n_pos * row
    _sync()
    plane = cap * row
    for w, t in ((0, pool.k[layer]), (1, pool.v[layer])):
        got = host(t)
        ref = oracle.kv_append_copy(np.zeros(0, np.uint16 if dt == "bf16" else np.float32), vals[w].ravel(), dt)
        assert np.array_equal(got[slot * plane:slot * plane + n_pos * row], ref)
        rest = np.concatenate([got[:slot * plane], got[slot * plane + n_pos * row:]])
        old = before[(layer, w)]
        assert np.array_equal(rest, np.concatenate([old[:slot * plane], old[slot * plane + n_pos * row:]]))
    for l in range(n_layer):
        if l != layer:
            assert np.array_equal(host(pool.k[l]), before[(l, 0)]) and np.array_equal(host(pool.v[l]), before[(l, 1)])
    # attention over the slot, at several context lengths, against the oracle on the oracle's own K/V
    for ctx in (1, 33, n_pos):
        q = synth.normal((H * hd,), 31, ctx, 1.0)
        kk = oracle.kv_append_copy(np.zeros(0, np.uint16 if dt == "bf16" else np.float32), vals[0][:ctx].ravel(), dt)
        vv = oracle.kv_append_copy(np.zeros(0, np.uint16 if dt == "bf16" else np.float32), vals[1][:ctx].ravel(), dt)
        out = torch.full((H * hd,), float("nan"), dtype=torch.float32, device="cuda")
        ws = llmk.workspace(llmk.gqa_attend_workspace_bytes(ctx, H, hd))
        assert llmk.gqa_attend(dev(q), pool, layer, slot, ctx, H, out, ws) == llmk.OK
        _sync()
        ref = oracle.attend_f32(q, kk.reshape(ctx, Hkv, hd), vv.reshape(ctx, Hkv, hd), ctx, H, Hkv, hd)
        assert rel_err(host(out), ref) <= TOL, ctx
    # more positions than the records hold is refused
    ws = llmk.workspace(llmk.gqa_attend_workspace_bytes(n_pos + 1, H, hd))
    out = torch.zeros(H * hd, dtype=torch.float32, device="cuda")
    assert llmk.gqa_attend(dev(q), pool, layer, slot, n_pos + 1, H, out, ws) == 566


# ---------------------------------------------------------------------------------------------
# argmax
# ---------------------------------------------------------------------------------------------

def run_argmax(logits_np, rows, n):
    lg = dev(logits_np.astype(np.float32).ravel())
    tok = torch.full((rows,), -5, dtype=torch.int32, device="cuda")
    val = torch.zeros(rows, dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.argmax_workspace_bytes(rows, n))
    assert llmk.argmax(lg, rows, n, tok, val, ws) == llmk.OK
    _sync()
    return host(tok), host(val)


def test_argmax_examples():
    g = golden("argmax_examples.json")
    for case in g["cases"]:
        row = np.array(case["logits"], np.float32)
        tok, val = run_argmax(row, 1, row.size)
        assert tok[0] == case["token_id"]
        if "logit" in case:
            assert val[0] == case["logit"]
    n, at = g["wide_row"]["n"], g["wide_row"]["planted_max_at"]
    row = synth.normal((n,), 10, 0, 3.0)
    row[at] = row.max() + 1.0
    assert run_argmax(row, 1, n)[0][0] == at


@pytest.mark.parametrize("seed", range(8))
def test_argmax_planted_ties_bit_exact(seed):
    V = 128256
    row = synth.normal((V,), 30 + seed, 0, 3.0)
    m = float(row.max()) + 0.5
    bpr_slice = (V + 63) // 64          # the library's per-workgroup slice at this width
    plants = [[7, 8], [bpr_slice - 1, bpr_slice], [0, V - 1], [V - 2, V - 1], [63, 64], [1000, 90000]]
    ties = plants[seed % len(plants)]
    for i in ties:
        row[i] = m
    tok, val = run_argmax(row, 1, V)
    ref_tok, ref_val = oracle.argmax(row)
    assert tok[0] == ref_tok == min(ties) and val[0] == ref_val


def test_argmax_signed_zero_nan_and_rows():
    rows = np.full((4, 1000), -1.0, np.float32)
    rows[0, [10, 20]] = [-0.0, 0.0]
    rows[1, [10, 20]] = [0.0, -0.0]
    rows[2, [5, 700, 900]] = [np.nan, 3.0, np.nan]
    rows[3, :] = -np.inf
    tok, _ = run_argmax(rows, 4, 1000)
    assert tok.tolist() == [oracle.argmax(r)[0] for r in rows] == [10, 10, 5, 0]


# ---------------------------------------------------------------------------------------------
# transpose (the one-time repacking into output-major weights)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("rows,cols,dt", [(1, 1, "f32"), (3, 5, "f32"), (65, 130, "bf16"), (4096, 14336, "bf16"),
                                          (1000, 24, "f32")])
def test_transpose_bit_exact(rows, cols, dt):
    a = synth.normal((rows, cols), 40, rows + cols, 1.0, dt)
    src = dev(a)
    dst = torch.empty_like(src)
    assert llmk.transpose(src, dst, rows, cols) == llmk.OK
    _sync()
    assert np.array_equal(host(dst).reshape(cols, rows), a.T)


# ---------------------------------------------------------------------------------------------
# the in-place append's cost shape
# ---------------------------------------------------------------------------------------------

def test_kv_append_cost_is_flat_in_the_cache_length():
    """Appending one decode token's row (1,024 elements) in place costs the same per element whether the cache
    holds 2,048 or 133,120 elements ("LLM inference kernels", "The hot loop doesn't call kv_cache_append_flat":
    the copying append grows with the cache, the in-place one does not; the gate allows 3x)."""
    cache = torch.zeros(140000, dtype=torch.bfloat16, device="cuda")
    newv = dev(synth.normal((1024,), 14, 0, 1.0))
    stream = torch.cuda.current_stream()
    per = {}
    for filled in (2048, 133120):
        for _ in range(5):
            assert llmk.kv_append_flat(cache, filled, filled, newv)[0] == llmk.OK
        _sync()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(400):
            assert llmk.kv_append_flat(cache, filled, filled, newv)[0] == llmk.OK
        e1.record(stream)
        _sync()
        per[filled] = e0.elapsed_time(e1) / 400 / 1024
    say(f"append per element: {per[2048] * 1e6:.3f} ns at 2,048, {per[133120] * 1e6:.3f} ns at 133,120")
    assert per[133120] <= 3.0 * per[2048]
