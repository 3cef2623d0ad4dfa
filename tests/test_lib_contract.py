"""The C-ABI library without a GPU: it loads, exports every symbol include/llmk.h declares, and every
host-side refusal returns the status the oracle's independent contract expects (CPU only).

Refusals are checked with stand-in pointers: the library validates every argument before its first
HIP call, so a refused call never touches them. Calls the oracle expects to succeed are not made here
(they would launch kernels); the GPU tests cover them. On a machine with a visible GPU the stand-in
pointer tests are skipped, so a library bug can never launch a kernel on them.
"""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

from oracle import contract
from tests.conftest import ROOT, golden

llmk = pytest.importorskip("autoregressive_decode_step_amd")

FAKE = 0x1000  # a non-null stand-in; never dereferenced by a refused call


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


no_gpu = pytest.mark.skipif(_gpu_visible(), reason="stand-in pointers are only safe without a GPU")


def test_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "llmk.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(llmk_\w+)\s*\(", header, flags=re.M))
    assert len(declared) >= 20
    lib = ctypes.CDLL(llmk.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), f"{name} declared in llmk.h but not exported"
    assert declared == set(llmk.EXPORTED)


def test_status_names_match_pages_and_oracle():
    g = golden("contract_examples.json")
    for code, name in g["status_table"].items():
        assert llmk.status_name(int(code)) == name
    for code in range(555, 585):
        assert llmk.status_name(code) == contract.status_name(code)
    assert llmk.status_name(-7) == contract.status_name(g["fallback_name_code"])


def test_page_contract_examples():
    g = golden("contract_examples.json")
    for case in g["residual_dims_check"]:
        assert llmk.residual_dims_check(*case["args"]) == case["status"]


VALS = [-1, 0, 1, 2, 3, 6, (1 << 24), (1 << 24) + 1]


def test_dims_checks_agree_with_oracle():
    for n, la, lb in itertools.product(VALS, repeat=3):
        assert llmk.residual_dims_check(n, la, lb) == contract.residual_dims_check(n, la, lb)
        assert llmk.argmax_dims_check(n, la) == contract.argmax_dims_check(n, la)
    for c, lc, nn, ln in itertools.product([-1, 0, 3, 6, (1 << 24) + 1], [0, 3, 6], [-1, 0, 1, 3], [0, 1, 3]):
        assert llmk.kv_append_dims_check(c, lc, nn, ln) == contract.kv_append_dims_check(c, lc, nn, ln)
    for m, n in itertools.product([-1, 0, 2, 3, (1 << 24) + 1], repeat=2):
        for la, lx in itertools.product([0, 6, m * n], [0, 2, m]):
            assert llmk.gemv_dims_check(m, n, la, lx) == contract.gemv_dims_check(m, n, la, lx)


def _nz(flag):
    return FAKE if flag else None


@no_gpu
def test_gemv_t_refusals():
    L = llmk.lib
    cases = 0
    for a, x, y, ws in itertools.product([True, False], repeat=4):
        for dt, m, n in itertools.product([0, 1, 5], [0, 2, (1 << 24) + 1], [3, -1]):
            for la, lx, ly in itertools.product([6, 5], [2, 1], [3, 4]):
                exp = contract.gemv_t(a, la, dt, x, lx, m, n, y, ly, ws)
                if exp == contract.OK:
                    continue
                got = L.llmk_gemv_t(_nz(a), la, dt, _nz(x), lx, m, n, _nz(y), ly, _nz(ws), 1 << 30, None)
                assert got == exp, (a, x, y, ws, dt, m, n, la, lx, ly)
                cases += 1
    assert cases > 100
    # a workspace shorter than the library asks for
    need = llmk.gemv_t_workspace_bytes(4096, 4096, 1)
    assert need > 0
    assert L.llmk_gemv_t(FAKE, 4096 * 4096, 1, FAKE, 4096, 4096, 4096, FAKE, 4096, FAKE, need - 1, None) == 578


@no_gpu
def test_elementwise_refusals():
    L = llmk.lib
    for a, b, o in itertools.product([True, False], repeat=3):
        for n, la, lb, lo in itertools.product([0, 4, (1 << 24) + 1], [4, 3], [4, 5], [4, 2]):
            exp = contract.residual_add(a, la, b, lb, n, o, lo)
            if exp != contract.OK:
                assert L.llmk_residual_add(_nz(a), la, _nz(b), lb, n, _nz(o), lo, None) == exp
            exp = contract.silu_mul(a, la, b, lb, n, o, lo)
            if exp != contract.OK:
                assert L.llmk_silu_mul(_nz(a), la, _nz(b), lb, n, _nz(o), lo, None) == exp
    for r, x, g, h in itertools.product([True, False], repeat=4):
        for rows, n, eps in itertools.product([0, 2], [0, 8], [1e-5, 0.0, float("nan")]):
            for lr, lx, lg, lh in itertools.product([16, 15], [16, 3], [8, 7], [16, 1]):
                exp = contract.add_rmsnorm(r, lr, x, lx, g, lg, rows, n, eps, h, lh)
                if exp != contract.OK:
                    got = L.llmk_add_rmsnorm(_nz(r), lr, _nz(x), lx, _nz(g), lg, rows, n, eps, _nz(h), lh, None)
                    assert got == exp, (r, x, g, h, rows, n, eps, lr, lx, lg, lh)


@no_gpu
def test_rope_refusals():
    L = llmk.lib
    for t, mp, hd, base in itertools.product([True, False], [0, 10], [0, 3, 8, 512], [1e4, 1.0, float("inf")]):
        for lt in (mp * hd, 5):
            exp = contract.rope_table_init(t, lt, mp, hd, base)
            if exp != contract.OK:
                assert L.llmk_rope_table_init(_nz(t), lt, mp, hd, base, None) == exp
    for q, k, tab in itertools.product([True, False], repeat=3):
        for rows, nq, nk, hd, pos, layout in itertools.product([0, 2], [0, 4], [-1, 0, 2], [6, 7], [True, False],
                                                               [0, 1, 2]):
            for lq, lk, lt, lp in itertools.product([rows * nq * hd, 1], [rows * max(nk, 0) * hd, 1], [10 * hd, 3],
                                                    [rows, 3]):
                exp = contract.rope(q, lq, k, lk, rows, nq, nk, hd, pos, lp, tab, lt, 10, layout)
                if exp != contract.OK:
                    got = L.llmk_rope(_nz(q), lq, _nz(k), lk, rows, nq, nk, hd, _nz(pos), lp, _nz(tab), lt, 10,
                                      layout, None)
                    assert got == exp, (q, k, tab, rows, nq, nk, hd, pos, layout, lq, lk, lt, lp)


@no_gpu
def test_kv_append_refusals():
    L = llmk.lib
    out = ctypes.c_int64(-7)
    for c, nv, dt in itertools.product([True, False], [True, False], [0, 1, 2]):
        for cap, cl, lc, nn, ln in itertools.product([0, 9, 8], [-1, 0, 6], [6, 5], [0, 3], [3, 2]):
            exp = contract.kv_append_flat(c, cap, dt, cl, lc, nv, ln, nn)
            if exp != contract.OK:
                got = L.llmk_kv_append_flat(_nz(c), cap, dt, cl, lc, _nz(nv), ln, nn, ctypes.byref(out), None)
                assert got == exp, (c, nv, dt, cap, cl, lc, nn, ln)
                assert out.value == -7  # untouched on refusal


class _FakePool:
    """A pool descriptor over fake (never dereferenced) device addresses, for host-only checks."""

    def __init__(self, n_layer=2, n_slots=3, capacity=8, n_kv=2, head_dim=4, dtype=0, arrays=True, buffers=True,
                 records=True, paged=False, bt=64, n_blocks=4, max_blocks=None, parrays=True):
        self.fields = dict(n_layer=n_layer, n_slots=n_slots, capacity=capacity, n_kv=n_kv, head_dim=head_dim,
                           dtype=dtype, arrays=arrays, buffers=buffers, records=records)
        nl = max(0, min(n_layer, 4))
        ptrs = [FAKE] * nl
        if not buffers and nl:
            ptrs[-1] = FAKE + 2   # a misaligned layer buffer
        self.kp = (ctypes.c_void_p * max(nl, 1))(*ptrs)
        self.vp = (ctypes.c_void_p * max(nl, 1))(*([FAKE] * nl))
        ns = max(0, min(n_slots, 8))
        self.slot_len = np.full(max(ns, 1), 5, dtype=np.int64)
        self.len_k = np.full((max(nl, 1), max(ns, 1)), 7, dtype=np.int64)
        self.len_v = np.full((max(nl, 1), max(ns, 1)), 7, dtype=np.int64)
        P = ctypes.POINTER(ctypes.c_int64)
        self.struct = llmk.PoolStruct(self.kp if arrays else None, self.vp, n_layer, n_slots, capacity, n_kv,
                                      head_dim, dtype, self.slot_len.ctypes.data_as(P),
                                      self.len_k.ctypes.data_as(P) if records else None,
                                      self.len_v.ctypes.data_as(P) if records else None)
        if paged:
            mb = -(-capacity // bt) if max_blocks is None else max_blocks
            self.fields["pages"] = dict(block_tokens=bt, n_blocks=n_blocks, max_blocks=mb, arrays=parrays)
            self.table_h = np.full((max(ns, 1), max(min(mb, 64), 1)), 9, dtype=np.int32)
            self.refcount = np.full(max(min(n_blocks, 64), 1), 9, dtype=np.int32)
            P32 = ctypes.POINTER(ctypes.c_int32)
            self.pages = llmk.PagesStruct(bt, n_blocks, mb, FAKE if parrays else None,
                                          self.table_h.ctypes.data_as(P32), self.refcount.ctypes.data_as(P32), 5)
            self.struct.pages = ctypes.pointer(self.pages)


POOL_CASES = [dict(), dict(arrays=False), dict(buffers=False), dict(dtype=3), dict(n_layer=0), dict(n_slots=-1),
              dict(capacity=0), dict(head_dim=(1 << 24) + 1), dict(n_kv=0, buffers=False), dict(records=False),
              dict(dtype=2), dict(dtype=2, head_dim=16), dict(dtype=2, head_dim=16, buffers=False),
              dict(dtype=2, head_dim=24, buffers=False)]
# paged pools: good ones, and one bad field each
PAGED_CASES = [dict(paged=True), dict(paged=True, capacity=130, bt=64, n_blocks=7), dict(paged=True, bt=32),
               dict(paged=True, bt=96), dict(paged=True, bt=131072), dict(paged=True, max_blocks=2),
               dict(paged=True, n_blocks=0), dict(paged=True, n_blocks=(1 << 24) + 1), dict(paged=True, parrays=False),
               dict(paged=True, n_slots=-1), dict(paged=True, capacity=1 << 24, n_slots=100),
               dict(paged=True, buffers=False, bt=32)]


@no_gpu
def test_kv_pool_init():
    for c in POOL_CASES + PAGED_CASES:
        fp = _FakePool(**c)
        exp = contract.kv_pool_init(fp.fields)
        got = llmk.lib.llmk_kv_pool_init(ctypes.byref(fp.struct))
        assert got == exp, c
        if got == contract.OK:   # every record of every slot marked empty
            assert not fp.slot_len.any() and (not c.get("records", True) or not (fp.len_k.any() or fp.len_v.any()))
            if c.get("paged"):   # no block held, every block free
                assert (fp.table_h == -1).all() and not fp.refcount.any() and fp.pages.n_free == fp.pages.n_blocks
        else:                    # refused: records untouched
            assert (fp.slot_len == 5).all()
            if c.get("paged"):
                assert (fp.table_h == 9).all() and fp.pages.n_free == 5
    assert llmk.lib.llmk_kv_pool_init(None) == contract.kv_pool_init(None) == 578


@no_gpu
def test_pool_append_and_attend_refusals():
    L = llmk.lib
    for c in POOL_CASES:
        for layer, slot, which, cl, nn, ln, rec in itertools.product([0, 2], [1, 3], [0, 2], [-1, 7, 6], [0, 2],
                                                                      [2, 1], [7]):
            fp = _FakePool(**c)
            exp, _, _ = contract.kv_append(fp.fields, layer, slot, which, cl, rec, True, ln, nn)
            if exp == contract.OK:
                continue   # would launch
            nl, off = ctypes.c_int64(-7), ctypes.c_int64(-7)
            got = L.llmk_kv_append(ctypes.byref(fp.struct), layer, slot, which, cl, FAKE, ln, nn, ctypes.byref(nl),
                                   ctypes.byref(off), None)
            assert got == exp, (c, layer, slot, which, cl, nn, ln)
            assert nl.value == -7 and off.value == -7 and (fp.len_k == 7).all() and (fp.len_v == 7).all()
    # overrun of the slot's region: capacity 8 positions x 2 heads x 4 = 64 elements, 7 filled
    fp = _FakePool()
    assert contract.kv_append(fp.fields, 0, 0, 0, 7, 7, True, 58, 58)[0] == contract.CAPACITY
    assert L.llmk_kv_append(ctypes.byref(fp.struct), 0, 0, 0, 7, FAKE, 58, 58, None, None, None) == contract.CAPACITY
    assert L.llmk_kv_append(ctypes.byref(fp.struct), 0, 0, 0, 7, None, 2, 2, None, None, None) == contract.INVALID
    for c in POOL_CASES:
        for layer, slot, ctx, H, lq, lo in itertools.product([0, 2], [0, 3], [0, 1, 2, 9], [4, 3, 32], [16, 5],
                                                             [16, 6]):
            fp = _FakePool(**c)
            rec = 7 if c.get("records", True) else None
            exp = contract.gqa_attend(True, lq, fp.fields, layer, slot, ctx, H, True, lo, rec, rec)
            if exp == contract.OK:
                continue
            got = L.llmk_gqa_attend(FAKE, lq, ctypes.byref(fp.struct), layer, slot, ctx, H, FAKE, lo, FAKE, 1 << 30,
                                    None)
            assert got == exp, (c, layer, slot, ctx, H, lq, lo)


@no_gpu
def test_attend_and_argmax_refusals():
    L = llmk.lib
    for ctx, H, Hkv, hd, dt in itertools.product([0, 5], [4, 6], [2, 4, 3], [4, 6, 512], [0, 1, 7]):
        for lq, lc, lo in itertools.product([H * hd, 1], [ctx * Hkv * hd, 2], [H * hd, 3]):
            exp = contract.gqa_attend_flat(True, lq, True, True, lc, dt, ctx, H, Hkv, hd, True, lo)
            if exp != contract.OK:
                got = L.llmk_gqa_attend_flat(FAKE, lq, FAKE, FAKE, lc, dt, ctx, H, Hkv, hd, FAKE, lo, FAKE, 1 << 30,
                                             None)
                assert got == exp, (ctx, H, Hkv, hd, dt, lq, lc, lo)
    for rows, n, ll in itertools.product([0, 1, 3], [0, 7], [21, 7, 0]):
        exp = contract.argmax(True, ll, rows, n, True)
        if exp != contract.OK:
            assert L.llmk_argmax(FAKE, ll, rows, n, FAKE, None, FAKE, 1 << 30, None) == exp
    assert L.llmk_argmax(None, 7, 1, 7, FAKE, None, FAKE, 1 << 30, None) == 578
    need = llmk.argmax_workspace_bytes(1, 128256)
    assert L.llmk_argmax(FAKE, 128256, 1, 128256, FAKE, None, FAKE, need - 1, None) == 578


@no_gpu
def test_sample_refusals():
    L = llmk.lib
    nan = float("nan")
    cases = itertools.product([0, 1, 3], [0, 7, 2000], [0, 1], [-1.0, nan, 0.0, 0.7], [0, 1, 5, 1024, 1025],
                              [0.0, 0.5, 1.0, 1.5], [0, 1, 3])
    for rows, n, bad_len, t, k, p, lu in cases:
        ll = rows * n + bad_len
        exp = contract.sample(True, ll, rows, n, t, k, p, True, lu, True)
        if exp != contract.OK:
            got = L.llmk_sample(FAKE, ll, rows, n, t, k, p, FAKE, lu, FAKE, FAKE, 1 << 40, None)
            assert got == exp, (rows, n, bad_len, t, k, p, lu)
    for null in range(3):
        ptrs = [FAKE, FAKE, FAKE]
        ptrs[null] = None
        assert L.llmk_sample(ptrs[0], 7, 1, 7, 1.0, 0, 1.0, ptrs[1], 1, ptrs[2], FAKE, 1 << 40, None) == 578
    rows = contract.SAMPLE_MAX_ROWS + 1
    assert L.llmk_sample(FAKE, rows * 9, rows, 9, 1.0, 3, 1.0, FAKE, rows, FAKE, FAKE, 1 << 40, None) == \
        contract.sample(True, rows * 9, rows, 9, 1.0, 3, 1.0, True, rows, True) == contract.TOO_LARGE
    # a call that needs a workspace refuses none, a short one and a misaligned one
    v = 128256
    need = llmk.sample_workspace_bytes(2, v, 1.0, 50)
    assert need > 0
    exp = contract.sample(True, 2 * v, 2, v, 1.0, 50, 0.9, True, 2, True, ws_short=True)
    for ws, n_ws in [(None, 0), (FAKE, need - 1), (FAKE + 8, need)]:
        assert L.llmk_sample(FAKE, 2 * v, 2, v, 1.0, 50, 0.9, FAKE, 2, FAKE, ws, n_ws, None) == exp == 578


def test_sample_workspace_sizes():
    # G * k candidates of 8 bytes and G slice maxima of 4 bytes per row: wave slices of 1,024 logits while
    # G * k <= 8,192, else of 2,048, else block slices of 16,384 under the same bound, else the one-workgroup
    # form with no workspace
    ws = llmk.sample_workspace_bytes
    assert ws(1, 128256, 1.0, 50) == 126 * (50 * 8 + 4)          # 126 wave slices of 1,024
    assert ws(1, 128256, 1.0, 65) == 126 * (65 * 8 + 4)
    assert ws(1, 128256, 1.0, 130) == 63 * (130 * 8 + 4)         # 126 * 130 > 8192: 63 slices of 2,048
    assert ws(2, 128256, 1.0, 131) == 2 * 8 * (131 * 8 + 4)      # 63 * 131 > 8192: 8 block slices
    assert ws(3, 128256, 0.7, 1024) == 3 * 8 * (1024 * 8 + 4)
    assert ws(1, 128256, 0.0, 0) == 126 * (1 * 8 + 4)            # greedy keeps one survivor
    assert ws(1, 5000, 1.0, 1000) == 5 * (1000 * 8 + 4)
    assert ws(1, 151936, 1.0, 1024) == 0                   # 10 block slices * 1024 > 8192: one workgroup
    assert ws(1, 2048, 1.0, 3) == 2 * (3 * 8 + 4)
    assert ws(1, 1024, 1.0, 3) == 0                        # one slice: one workgroup
    assert ws(0, 7, 1.0, 3) == -561 and ws(1, 5000, 1.0, 0) == -564


def test_kv_slot_offset_closed_form():
    import numpy as np

    class FakePool:
        pass

    n_slots, cap, n_kv, hd = 3, 10, 2, 4
    ks = (ctypes.c_void_p * 1)(FAKE)
    lens = np.zeros(n_slots, np.int64)
    ps = llmk.PoolStruct(ks, ks, 1, n_slots, cap, n_kv, hd, 0, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    fp = FakePool()
    fp.struct = ps
    for slot, pos, g in itertools.product([-1, 0, 2, 3], [-1, 0, 9, 10], [-1, 0, 1, 2]):
        exp_st, exp_off = contract.kv_slot_offset(n_slots, cap, n_kv, hd, slot, pos, g)
        st, off = llmk.kv_slot_offset(fp, slot, pos, g)
        assert st == exp_st
        if st == contract.OK:
            assert off == exp_off


def _cfg_kwargs(**over):
    kw = dict(vocab=40, d=16, n_layer=2, n_head=4, n_kv=2, head_dim=4, hidden=24, max_seq=64, eps=1e-5,
              rope_base=1e4, rope_layout=0, w_dtype=0, kv_dtype=0)
    kw.update(over)
    return kw


def test_config_checks_agree_with_oracle():
    variants = [dict(), dict(test_flags=1), dict(test_flags=2), dict(test_flags=-1), dict(vocab=0),
                dict(d=(1 << 24) + 1), dict(n_head=6), dict(n_kv=3), dict(head_dim=6),
                dict(head_dim=512), dict(n_head=32, n_kv=2), dict(hidden=22), dict(w_dtype=1), dict(w_dtype=3),
                dict(rope_layout=2), dict(eps=0.0), dict(rope_base=1.0), dict(max_seq=-4), dict(kv_dtype=1),
                dict(d=12, w_dtype=0), dict(d=24, w_dtype=1), dict(kv_dtype=2), dict(kv_dtype=3),
                dict(kv_dtype=2, head_dim=16), dict(kv_dtype=2, head_dim=16, step_path=2),
                dict(kv_dtype=2, head_dim=16, step_path=1, w_dtype=1)]
    for v in variants:
        kw = _cfg_kwargs(**v)
        cfg = llmk.make_config(**kw)
        got = llmk.decode_workspace_bytes(cfg, 1)
        exp = contract.config_check(**kw)
        if exp == contract.OK:
            assert got > 0, v
        else:
            assert got == -exp, v


@no_gpu
def test_decode_step_refusals():
    import numpy as np
    kw = _cfg_kwargs()
    cfg = llmk.make_config(**kw)
    d, qd, kvd, F, V, L = 16, 16, 8, 24, 40, 2
    lens = [d * qd, d * kvd, d * kvd, qd * d, d * F, d * F, F * d, d, d]
    FA = 0x10000  # 16-byte aligned stand-in

    def model(bad_len=False, null=False):
        arr = (llmk.Tensor * (L * 9))()
        for l in range(L):
            for t in range(9):
                arr[l * 9 + t] = llmk.Tensor(None if (null and l == 1 and t == 3) else FA,
                                             lens[t] + (1 if (bad_len and l == 1 and t == 5) else 0))
        m = llmk.ModelStruct(llmk.Tensor(FA, V * d), llmk.Tensor(FA, V * d), llmk.Tensor(FA, d),
                             llmk.Tensor(FA, 64 * 4), arr)
        return m, arr

    ws_need = llmk.decode_workspace_bytes(cfg, 1)

    def call(m, n_slots=2, cap=32, slot=0, slot_len=0, token=0, pos=0, logits=False, len_logits=V, hidden=False,
             len_hidden=L * d, ws_len=None, pool_nkv=2):
        ks = (ctypes.c_void_p * L)(FA, FA)
        sl = np.full(max(n_slots, 1), slot_len, np.int64)
        ps = llmk.PoolStruct(ks, ks, L, n_slots, cap, pool_nkv, 4, 0, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return llmk.lib.llmk_decode_step(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), slot, token, pos,
                                         FA if logits else None, len_logits, FA, FA if hidden else None, len_hidden,
                                         FA, ws_need if ws_len is None else ws_len, None)

    good, _a = model()
    cases = [
        (dict(slot=2), dict(slot=2, n_slots=2)),
        (dict(token=40), dict(token=40)),
        (dict(token=-1), dict(token=-1)),
        (dict(pos=64, slot_len=64, cap=128), dict(pos=64, slot_len=64, capacity=128)),
        (dict(pos=3, slot_len=2), dict(pos=3, slot_len=2)),
        (dict(pos=32, slot_len=32, cap=32), dict(pos=32, slot_len=32, capacity=32)),
        (dict(logits=True, len_logits=39), dict(logits=True, len_logits=39)),
        (dict(hidden=True, len_hidden=31), dict(hidden=True, len_hidden=31)),
        (dict(ws_len=ws_need - 1), dict(ws_short=True)),
        (dict(n_slots=0), dict(n_slots=0, pool_dims_bad=True)),
        (dict(pool_nkv=4), dict(pool_ok=False)),
    ]
    for call_kw, exp_kw in cases:
        base = dict(n_slots=2, capacity=32, slot=0, slot_len=0, token=0, pos=0)
        base.update(exp_kw)
        exp = contract.decode_step(kw, **base)
        assert exp != contract.OK
        assert call(good, **call_kw) == exp, call_kw
    bad, _b = model(bad_len=True)
    assert call(bad) == contract.decode_step(kw, lens_ok=False) == 576
    nul, _c = model(null=True)
    assert call(nul) == contract.decode_step(kw, tensors_ok=False) == 578

    # the kernel-timing aid refuses exactly as the step does, then checks its own arguments
    def kt(kernel=3, reps=4, ms=True, token=0):
        ks = (ctypes.c_void_p * L)(FA, FA)
        sl = np.zeros(2, np.int64)
        ps = llmk.PoolStruct(ks, ks, L, 2, 32, 2, 4, 0, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        out = ctypes.c_float(0.0)
        return llmk.lib.llmk_decode_kernel_time(ctypes.byref(cfg), ctypes.byref(good), ctypes.byref(ps), 0, token, 0,
                                                kernel, reps, FA, ctypes.byref(out) if ms else None, FA, ws_need,
                                                None)
    assert kt(token=40) == contract.decode_step(kw, token=40) == 572
    assert kt(ms=False) == 578
    assert kt(kernel=6) == 578 and kt(kernel=-1) == 578
    assert kt(reps=0) == 561
    assert kt(reps=65) == 564


@no_gpu
def test_decode_step_batch_refusals():
    import numpy as np
    d, qd, kvd, F, V, L = 16, 16, 8, 24, 40, 2
    lens = [d * qd, d * kvd, d * kvd, qd * d, d * F, d * F, F * d, d, d]
    FA = 0x10000

    def model_for(kw, bad_len=False):
        arr = (llmk.Tensor * (L * 9))()
        for l in range(L):
            for t in range(9):
                arr[l * 9 + t] = llmk.Tensor(FA, lens[t] + (1 if (bad_len and l == 1 and t == 2) else 0))
        return llmk.ModelStruct(llmk.Tensor(FA, V * d), llmk.Tensor(FA, V * d), llmk.Tensor(FA, d),
                                llmk.Tensor(FA, 64 * 4), arr), arr

    def run(kw, batch=2, slots=(0, 1), tokens=(0, 0), pos=(0, 0), slot_lens=(0, 0, 0), cap=32, n_slots=3,
            logits=False, len_logits=None, len_tokens=None, hidden=False, len_hidden=None, ws_short=False,
            n_steps=None, bad_len=False):
        cfg = llmk.make_config(**kw)
        m, _keep = model_for(kw, bad_len)
        ks = (ctypes.c_void_p * L)(FA, FA)
        sl = np.array(slot_lens, np.int64)
        ps = llmk.PoolStruct(ks, ks, L, n_slots, cap, 2, 4, kw["kv_dtype"],
                             sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        a_s, a_t, a_p = (np.array(v, np.int64) for v in (slots, tokens, pos))
        ws_need = llmk.decode_workspace_bytes(cfg, max(1, min(batch, 64)))
        ws = max(ws_need, 1) - (1 if ws_short else 0)
        if n_steps is None:
            return llmk.lib.llmk_decode_step_batch(
                ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), batch, a_s.ctypes.data, a_t.ctypes.data,
                a_p.ctypes.data, FA if logits else None, batch * V if len_logits is None else len_logits, FA,
                batch if len_tokens is None else len_tokens, FA if hidden else None,
                batch * L * d if len_hidden is None else len_hidden, FA, ws, None)
        return llmk.lib.llmk_decode_steps_batch(
            ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), batch, a_s.ctypes.data, a_t.ctypes.data,
            a_p.ctypes.data, n_steps, FA, n_steps * batch if len_tokens is None else len_tokens, FA, ws, None)

    good = _cfg_kwargs(w_dtype=1, w_layout=1)
    cases = [
        (dict(batch=0), dict(batch=0)),
        (dict(batch=65, slots=tuple(range(65)), tokens=(0,) * 65, pos=(0,) * 65, slot_lens=(0,) * 70, n_slots=70),
         dict(batch=65)),
        (dict(slots=(0, 3)), dict(slots=(0, 3))),
        (dict(slots=(1, 1)), dict(slots=(1, 1))),
        (dict(tokens=(0, 40)), dict(tokens=(0, 40))),
        (dict(pos=(0, -1)), dict(pos=(0, -1))),
        (dict(pos=(0, 64), slot_lens=(0, 64, 0), cap=128), dict(pos=(0, 64), slot_lens={1: 64}, capacity=128)),
        (dict(pos=(0, 5), slot_lens=(0, 4, 0)), dict(pos=(0, 5), slot_lens={1: 4})),
        (dict(pos=(0, 32), slot_lens=(0, 32, 0), cap=32), dict(pos=(0, 32), slot_lens={1: 32}, capacity=32)),
        (dict(logits=True, len_logits=79), dict(logits=True, len_logits=79)),
        (dict(len_tokens=3), dict(len_tokens=3)),
        (dict(hidden=True, len_hidden=63), dict(hidden=True, len_hidden=63)),
        (dict(ws_short=True), dict(ws_short=True)),
        (dict(bad_len=True), dict(lens_ok=False)),
        (dict(n_steps=0), dict(n_steps=0)),
        (dict(n_steps=40, pos=(0, 0)), dict(n_steps=40)),
        (dict(n_steps=3, len_tokens=5), dict(n_steps=3, len_tokens=5)),
    ]
    for call_kw, exp_kw in cases:
        base = dict(batch=2, n_slots=3, capacity=32, slots=(0, 1), tokens=(0, 0), pos=(0, 0))
        base.update({k: v for k, v in call_kw.items() if k in ("batch", "slots", "tokens", "pos")})
        base.update(exp_kw)
        if "n_slots" in call_kw:
            base["n_slots"] = call_kw["n_slots"]
        exp = contract.decode_step_batch(good, **base)
        assert exp != contract.OK, call_kw
        assert run(good, **call_kw) == exp, (call_kw, exp)
    # the batched path needs bf16 output-major weights
    for bad in (_cfg_kwargs(w_dtype=1, w_layout=0), _cfg_kwargs(w_dtype=0, w_layout=1)):
        exp = contract.decode_step_batch(bad, batch=2, n_slots=3, capacity=32, slots=(0, 1), tokens=(0, 0), pos=(0, 0),
                                         batch_weights_ok=False)
        assert run(bad) == exp == 578
        assert llmk.decode_workspace_bytes(llmk.make_config(**bad), 2) == -578


@no_gpu
def test_prefill_refusals():
    import numpy as np
    d, qd, kvd, F, V, L = 16, 16, 8, 24, 40, 2
    lens = [d * qd, d * kvd, d * kvd, qd * d, d * F, d * F, F * d, d, d]
    FA = 0x10000

    def model_for(bad_len=False):
        arr = (llmk.Tensor * (L * 9))()
        for l in range(L):
            for t in range(9):
                arr[l * 9 + t] = llmk.Tensor(FA, lens[t] + (1 if (bad_len and l == 1 and t == 2) else 0))
        return llmk.ModelStruct(llmk.Tensor(FA, V * d), llmk.Tensor(FA, V * d), llmk.Tensor(FA, d),
                                llmk.Tensor(FA, 64 * 4), arr), arr

    def run(kw, n=3, slot=1, tokens=None, pos0=0, slot_lens=(0, 0, 0), cap=32, n_slots=3, len_tokens=None,
            logits=False, len_logits=V, hidden=False, len_hidden=L * d, ws_short=False, bad_len=False):
        cfg = llmk.make_config(**kw)
        m, _keep = model_for(bad_len)
        ks = (ctypes.c_void_p * L)(FA, FA)
        sl = np.array(slot_lens, np.int64)
        ps = llmk.PoolStruct(ks, ks, L, n_slots, cap, 2, 4, kw["kv_dtype"],
                             sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        tk = np.array(tokens if tokens is not None else [0] * max(n, 0), np.int64)
        need = llmk.prefill_workspace_bytes(cfg, max(n, 1))
        ws = max(need, 1) - (1 if ws_short else 0)
        return llmk.lib.llmk_prefill(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), slot, tk.ctypes.data, n,
                                     pos0, FA, n if len_tokens is None else len_tokens, FA if logits else None,
                                     len_logits, FA if hidden else None, len_hidden, FA, ws, None)

    good = _cfg_kwargs(w_dtype=1, w_layout=1)
    cases = [
        (dict(n=0), dict(n=0)),
        (dict(slot=3), dict(slot=3)),
        (dict(tokens=[0, 40, 0]), dict(tokens=[0, 40, 0])),
        (dict(pos0=-1), dict(pos0=-1)),
        (dict(n=3, pos0=62, slot_lens=(0, 62, 0), cap=128), dict(pos0=62, slot_len=62, capacity=128)),
        (dict(pos0=5, slot_lens=(0, 4, 0)), dict(pos0=5, slot_len=4)),
        (dict(pos0=30, slot_lens=(0, 30, 0), cap=32), dict(pos0=30, slot_len=30, capacity=32)),
        (dict(len_tokens=2), dict(len_tokens=2)),
        (dict(logits=True, len_logits=3 * V), dict(logits=True, len_logits=3 * V)),
        (dict(hidden=True, len_hidden=3 * L * d), dict(hidden=True, len_hidden=3 * L * d)),
        (dict(ws_short=True), dict(ws_short=True)),
        (dict(bad_len=True), dict(lens_ok=False)),
    ]
    for call_kw, exp_kw in cases:
        base = dict(n=call_kw.get("n", 3), n_slots=3, capacity=32, slot=1, tokens=call_kw.get("tokens", [0] * 3))
        base.update(exp_kw)
        exp = contract.prefill(good, **base)
        assert exp != contract.OK, call_kw
        assert run(good, **call_kw) == exp, (call_kw, exp)
    for bad in (_cfg_kwargs(w_dtype=1, w_layout=0), _cfg_kwargs(w_dtype=0, w_layout=1)):
        exp = contract.prefill(bad, n=3, n_slots=3, capacity=32, slot=1, tokens=[0] * 3, batch_weights_ok=False)
        assert run(bad) == exp == 578
        assert llmk.prefill_workspace_bytes(llmk.make_config(**bad), 3) == -578
    # the profiled form refuses a missing or short phase buffer first, then as llmk_prefill
    cfg = llmk.make_config(**good)
    m, _keep = model_for()
    ks = (ctypes.c_void_p * L)(FA, FA)
    sl = np.zeros(3, np.int64)
    ps = llmk.PoolStruct(ks, ks, L, 3, 32, 2, 4, good["kv_dtype"], sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
    tk = np.zeros(3, np.int64)
    ms = (ctypes.c_float * 4)()
    prof = llmk.lib.llmk_prefill_profiled
    assert prof(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), 1, tk.ctypes.data, 3, 0, FA, 3, None, 4, FA,
                1 << 30, None) == 578
    assert prof(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), 1, tk.ctypes.data, 3, 0, FA, 3, ms, 3, FA,
                1 << 30, None) == 577
    assert prof(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), 3, tk.ctypes.data, 3, 0, FA, 3, ms, 4, FA,
                1 << 30, None) == contract.prefill(good, n=3, n_slots=3, capacity=32, slot=3, tokens=[0] * 3) == 575
    assert llmk.prefill_workspace_bytes(cfg, 0) == -561
    # 200 tokens are one chunk of 200 rows: the workspace holds its row buffers, its logits and hidden states
    assert llmk.prefill_workspace_bytes(cfg, 200) >= llmk.decode_workspace_bytes(cfg, 64) + 200 * (V + L * d) * 4


def test_q8_config_checks_agree_with_oracle():
    base = dict(vocab=40, d=128, n_layer=2, n_head=2, n_kv=1, head_dim=64, hidden=256, max_seq=64, w_dtype=2,
                w_layout=1)
    variants = [dict(), dict(w_layout=0), dict(step_path=2), dict(step_path=1), dict(hidden=200), dict(d=192),
                dict(head_dim=32, n_head=3, n_kv=1), dict(d=4096, hidden=14336, n_head=32, n_kv=8, head_dim=128),
                dict(hidden=16384), dict(hidden=16384 + 128), dict(d=1024, hidden=3072), dict(kv_dtype=2)]
    for v in variants:
        kw = _cfg_kwargs(**{**base, **v})
        cfg = llmk.make_config(**kw)
        got = llmk.decode_workspace_bytes(cfg, 1)
        exp = contract.config_check(**kw)
        if exp == contract.OK:
            assert got > 0, v
            # the batched path and prefill run bf16 weights only
            assert llmk.decode_workspace_bytes(cfg, 2) == -contract.INVALID, v
            assert llmk.prefill_workspace_bytes(cfg, 4) == -contract.INVALID, v
        else:
            assert got == -exp, v


def test_q8_pack_bytes_and_quantize_refusals():
    for rows, cols in ((1, 128), (3, 256), (128256, 4096), (0, 128), (4, 0), (4, 100), ((1 << 24) + 1, 128),
                       (2, (1 << 24) + 128)):
        assert llmk.q8_pack_bytes(rows, cols) == contract.q8_pack_bytes(rows, cols), (rows, cols)
    assert llmk.q8_pack_bytes(3, 256) == 3 * 256 + 4 * 3 * 2
    FA = 0x10000
    ok = dict(w=True, len_w=4 * 256, w_dtype=1, rows=4, cols=256, pack=True, len_pack=4 * 256 + 32)
    cases = [dict(), dict(w=False), dict(pack=False), dict(w_dtype=2), dict(w_dtype=-1), dict(rows=0), dict(cols=-128),
             dict(rows=(1 << 24) + 1), dict(cols=200, len_w=800), dict(len_w=4 * 256 - 1), dict(len_pack=4 * 256),
             dict(len_pack=4 * 256 + 33), dict(aligned=False, w_off=2), dict(aligned=False, pack_off=8),
             dict(aligned=False, pack_off=1, len_pack=7)]
    for c in cases:
        a = {**ok, **c}
        w_off, pack_off = a.pop("w_off", 0), a.pop("pack_off", 0)
        exp = contract.quantize_q8(**a)
        if exp == contract.OK:
            continue   # only refusals run here (no device)
        got = llmk.lib.llmk_quantize_q8(FA + w_off if a["w"] else None, a["len_w"], a["w_dtype"], a["rows"], a["cols"],
                                        FA + pack_off if a["pack"] else None, a["len_pack"], None)
        assert got == exp, c


@no_gpu
def test_q8_decode_model_lengths():
    import numpy as np
    kw = _cfg_kwargs(vocab=40, d=128, n_layer=2, n_head=2, n_kv=1, head_dim=64, hidden=256, max_seq=64, w_dtype=2,
                     w_layout=1)
    cfg = llmk.make_config(**kw)
    d, qd, kvd, F, V, L = 128, 128, 64, 256, 40, 2
    pb = contract.q8_pack_bytes
    lens = [pb(qd, d), pb(kvd, d), pb(kvd, d), pb(d, qd), pb(F, d), pb(F, d), pb(d, F), d, d]
    FA = 0x10000
    ws_need = llmk.decode_workspace_bytes(cfg, 1)

    def call(bad=None):
        arr = (llmk.Tensor * (L * 9))()
        for l in range(L):
            for t in range(9):
                arr[l * 9 + t] = llmk.Tensor(FA, lens[t] + (1 if bad == (l, t) else 0))
        out_len = pb(V, d) + (1 if bad == "out" else 0)
        emb_len = V * d + (1 if bad == "emb" else 0)
        m = llmk.ModelStruct(llmk.Tensor(FA, emb_len), llmk.Tensor(FA, out_len), llmk.Tensor(FA, d),
                             llmk.Tensor(FA, 64 * 64), arr)
        ks = (ctypes.c_void_p * L)(FA, FA)
        sl = np.zeros(2, np.int64)
        ps = llmk.PoolStruct(ks, ks, L, 2, 32, 1, 64, 0, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        # token 40 is out of range: every earlier check passed, nothing is launched
        return llmk.lib.llmk_decode_step(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), 0, 40, 0, None, V, FA,
                                         None, 0, FA, ws_need, None)
    assert call() == contract.decode_step(kw, token=40) == 572
    for bad in ((0, 0), (1, 6), (1, 3), "out", "emb"):
        assert call(bad) == contract.decode_step(kw, lens_ok=False) == 576, bad


@no_gpu
def test_decode_steps_sampled_refusals():
    import numpy as np
    kw = _cfg_kwargs()
    cfg = llmk.make_config(**kw)
    d, qd, kvd, F, V, L = 16, 16, 8, 24, 40, 2
    lens = [d * qd, d * kvd, d * kvd, qd * d, d * F, d * F, F * d, d, d]
    FA = 0x10000
    arr = (llmk.Tensor * (L * 9))()
    for l in range(L):
        for t in range(9):
            arr[l * 9 + t] = llmk.Tensor(FA, lens[t])
    m = llmk.ModelStruct(llmk.Tensor(FA, V * d), llmk.Tensor(FA, V * d), llmk.Tensor(FA, d), llmk.Tensor(FA, 64 * 4),
                         arr)
    ws_need = llmk.decode_workspace_bytes(cfg, 1)

    def call(n=4, token=0, draws=True, len_draws=None, T=1.0, k=0, p=1.0, sws=True, len_sws=1 << 20, ws_len=None):
        ks = (ctypes.c_void_p * L)(FA, FA)
        sl = np.zeros(2, np.int64)
        ps = llmk.PoolStruct(ks, ks, L, 2, 32, 2, 4, 0, sl.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)))
        return llmk.lib.llmk_decode_steps_sampled(ctypes.byref(cfg), ctypes.byref(m), ctypes.byref(ps), 0, token, 0, n,
                                                  T, k, p, FA if draws else None, n if len_draws is None else len_draws,
                                                  FA, n, FA, ws_need if ws_len is None else ws_len,
                                                  FA if sws else None, len_sws, None)
    base = dict(n_slots=2, capacity=32, slot=0, slot_len=0, token=0, pos=0)
    cases = [(dict(draws=False), dict(draws=False)), (dict(token=40), dict(token=40)), (dict(n=0), dict(n_steps=0)),
             (dict(n=40), dict(n_steps=40)), (dict(len_draws=3), dict(len_draws=3)), (dict(T=-1.0), dict(temperature=-1.0)),
             (dict(T=float("nan")), dict(temperature=float("nan"))), (dict(p=0.0), dict(top_p=0.0)),
             (dict(p=1.5), dict(top_p=1.5)), (dict(ws_len=ws_need - 1), dict(ws_short=True))]
    for call_kw, exp_kw in cases:
        e = dict(base)
        e.update(exp_kw)
        n = e.pop("n_steps", 4)
        exp = contract.decode_steps_sampled(kw, n_steps=n, **e)
        assert exp != contract.OK, call_kw
        assert call(**call_kw) == exp, (call_kw, exp)
    # a 40-entry vocabulary takes the one-workgroup sampler, which needs no workspace (sample_ws may be NULL);
    # the sampler-workspace refusal is checked on a vocabulary that needs one
    assert llmk.sample_workspace_bytes(1, V, 1.0, 0) == 0
    assert llmk.sample_workspace_bytes(1, 128256, 1.0, 50) > 0


@no_gpu
def test_paged_entry_points_pool_refusals():
    # every pool refusal of the paged-only entry points, and 578 for a pool without pages
    L = llmk.lib
    for c in POOL_CASES + PAGED_CASES:
        fp = _FakePool(**c)
        L.llmk_kv_pool_init(ctypes.byref(fp.struct))
        f, ps = fp.fields, ctypes.byref(fp.struct)
        exp = contract.kv_release(f, 1)
        if exp != contract.OK:
            assert L.llmk_kv_release(ps, 1) == exp, c
            assert L.llmk_kv_reserve(ps, 1, 0, 1, None) == contract.kv_reserve(f, 1, 0, 1) == exp, c
            assert L.llmk_kv_fork(ps, 0, 1, 1, None) == contract.kv_fork(f, 0, 1, 1) == exp, c
            adm = ctypes.c_int32(-7)
            assert L.llmk_kv_admit(ps, 3, ctypes.byref(adm)) == contract.kv_admit(f, 3)[0] == exp, c
            assert adm.value == -7
    for fn in (lambda: L.llmk_kv_release(None, 0), lambda: L.llmk_kv_reserve(None, 0, 0, 1, None),
               lambda: L.llmk_kv_fork(None, 0, 1, 1, None), lambda: L.llmk_kv_admit(None, 0, ctypes.byref(ctypes.c_int32()))):
        assert fn() == contract.INVALID
    fp = _FakePool(paged=True)
    assert L.llmk_kv_admit(ctypes.byref(fp.struct), 0, None) == contract.kv_admit(fp.fields, 0, admit=False)[0] == 578


def _paged_state():
    """A full paged pool (4 blocks of 64, 3 slots of up to 130 positions) and the oracle block manager in the
    same state: slot 0 holds blocks [0, 1] (100 positions), slot 1 [0, 2] (120, sharing block 0 with slot 0),
    slot 2 [3] (10)."""
    from oracle.paged import BlockManager
    fp = _FakePool(paged=True, capacity=130, bt=64, n_blocks=4)
    assert llmk.lib.llmk_kv_pool_init(ctypes.byref(fp.struct)) == contract.OK
    bm = BlockManager(3, 130, 4, 64)
    bm.table = [[0, 1, -1], [0, 2, -1], [3, -1, -1]]
    bm.ref = [2, 1, 1, 1]
    bm.length = [100, 120, 10]
    fp.table_h[:] = np.array(bm.table, dtype=np.int32)
    fp.refcount[:] = np.array(bm.ref, dtype=np.int32)
    fp.pages.n_free = bm.n_free()
    fp.slot_len[:] = bm.length
    fp.len_k[:] = fp.len_v[:] = np.array(bm.length) * 8
    return fp, bm


def _same(fp, bm):
    return (fp.table_h.tolist() == bm.table and fp.refcount.tolist() == bm.ref and fp.pages.n_free == bm.n_free()
            and fp.slot_len.tolist() == bm.length)


@no_gpu
def test_paged_block_manager_host_paths_match_oracle():
    """The library's host bookkeeping against the oracle's block manager wherever it needs no device work:
    reservations inside private blocks, refusals when full (nothing changes), release, admission, offsets."""
    L = llmk.lib
    fp, bm = _paged_state()
    ps = ctypes.byref(fp.struct)
    f = fp.fields
    # inside a private block: nothing to take (no device work), accepted
    for slot, b, e in [(0, 100, 101), (1, 120, 128), (2, 10, 64)]:
        st, copies = bm.reserve([(slot, b, e)])
        assert st == contract.OK and copies == []
        assert L.llmk_kv_reserve(ps, slot, b, e, None) == contract.kv_reserve(f, slot, b, e, 0, 0) == st
        assert _same(fp, bm)
    # a fresh block, a copy of shared block 0, both, past the capacity: refused, nothing changed
    for slot, b, e, need in [(1, 120, 129, 1), (0, 60, 61, 1), (0, 60, 130, 2), (2, 0, 131, 0)]:
        st, _ = bm.reserve([(slot, b, e)])
        assert st == contract.CAPACITY
        assert L.llmk_kv_reserve(ps, slot, b, e, None) == contract.kv_reserve(f, slot, b, e, need, 0) == st
        assert _same(fp, bm)
    # an append into a fresh block with none free: 571, records untouched
    st, nl, off = contract.kv_append(f, 0, 1, 0, 120 * 8, 120 * 8, True, 8 * 9, 8 * 9, need=1, n_free=0)
    assert st == contract.CAPACITY
    assert L.llmk_kv_append(ps, 0, 1, 0, 120 * 8, FAKE, 72, 72, None, None, None) == st
    assert _same(fp, bm) and fp.len_k[0, 1] == 960
    # attention over positions without a block: 573
    rec = 130 * 8
    exp = contract.gqa_attend(True, 16, f, 0, 2, 70, 4, True, 16, rec, rec, blocks_ok=False)
    fp.len_k[:] = fp.len_v[:] = rec
    assert L.llmk_gqa_attend(FAKE, 16, ps, 0, 2, 70, 4, FAKE, 16, FAKE, 1 << 30, None) == exp == contract.POSITION
    # fork refusals
    for src, dst, n, exp_args in [(0, 0, 5, {}), (0, 1, 5, dict(dst_len=120)), (0, 2, 5, dict(dst_len=10)),
                                  (0, 1, 0, {}), (0, 3, 5, {}), (1, 2, 121, dict(dst_len=10))]:
        exp = contract.kv_fork(f, src, dst, n, src_len=bm.length[src] if src < 3 else 0, **exp_args)
        assert exp != contract.OK
        assert L.llmk_kv_fork(ps, src, dst, n, None) == exp, (src, dst, n)
        assert _same(fp, bm)
    # release: slot 0 drops blocks 0 (still held by slot 1) and 1 (freed)
    bm.release(0)
    assert L.llmk_kv_release(ps, 0) == contract.kv_release(f, 0) == contract.OK
    assert _same(fp, bm) and fp.pages.n_free == 1 and not fp.len_k[:, 0].any()
    assert L.llmk_kv_release(ps, 3) == contract.kv_release(f, 3) == contract.SLOT
    # admission with one free block: an empty suffix fits (its headroom block), one more position does not
    for n in (0, 1, 64, 65):
        adm = ctypes.c_int32(-1)
        assert L.llmk_kv_admit(ps, n, ctypes.byref(adm)) == contract.OK
        assert (adm.value, contract.kv_admit(f, n, n_free=1)[1]) == (int(bm.admit(n)), int(bm.admit(n)))
    assert L.llmk_kv_admit(ps, -1, ctypes.byref(adm)) == contract.kv_admit(f, -1)[0] == contract.EMPTY
    # offsets through the table
    out = ctypes.c_int64(-1)
    for slot, pos, kvh in [(1, 0, 0), (1, 70, 1), (2, 5, 1), (0, 5, 0), (1, 129, 0)]:
        exp = contract.kv_slot_offset(3, 130, 2, 4, slot, pos, kvh, table=bm.table, block_tokens=64)
        assert L.llmk_kv_slot_offset(ps, slot, pos, kvh, ctypes.byref(out)) == exp[0], (slot, pos)
        if exp[0] == contract.OK:
            assert out.value == exp[1]
    assert contract.kv_slot_offset(3, 130, 2, 4, 1, 70, 1, table=bm.table, block_tokens=64) == \
        (contract.OK, (2 * 64 + 6) * 8 + 4)
