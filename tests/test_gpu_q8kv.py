"""The int8 K/V cache on the GPU against the oracle's int8 cache (MI355X only).

Format (the library's own; the pages name int8 K/V caches without fixing one): per (position, K/V head) row an
fp32 scale s = max|x| / 127 and codes rint(x / s) clamped to 127, the row standing for codes * s; each layer
buffer holds the codes, then the scales.

  - prefill of a 100-token prompt (rows rotated and quantized by the chunk's append, attention over the codes),
    then captured decode steps crossing tile boundaries, one kernel per operation: every greedy token equals the
    oracle's (teacher-forced on the GPU's inputs, its own int8 cache) or is a reported near-tie, the last
    prefill logits and every single step's logits and hidden states are within 2e-3, and the stored codes and
    scales equal the oracle's within the bar. A code may differ by one, never more, where the two sides' fp32
    values straddle a rounding boundary: with values agreeing to a relative e (1e-5 .. 1e-4 for fp32 sums of
    bf16 products), a code x / s about 40 on average sits within e * 40 of a half-integer for a fraction
    2 * 40 * e of the codes, about 0.1 .. 1 %; the count is reported and bounded by 2 %;
  - a batched step over three sequences with seeded int8 prefixes of different lengths, and its graph-replayed
    continuation, against the oracle row by row;
  - a paged int8 pool: a fork copies codes and scales on the first write, and the logits equal the contiguous
    pool's bit for bit;
  - llmk_gqa_attend over an int8 pool against the oracle's attention over what the rows stand for.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import TOL, dev, host, rel_err, say, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402

S = synth.Shape("int8 K/V test decoder bf16 (V512 d256 L2 H4/2 hd128 F512)", 512, 256, 2, 4, 2, 128, 512, 320,
                1e-5, 1e4, synth.ROPE_HALF_SPLIT, "bf16", "q8", 0.05)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def near_tie(logits, tol=TOL):
    s = np.sort(np.asarray(logits, np.float64))
    return (s[-1] - s[-2]) <= 2 * tol * np.max(np.abs(s))


def check_codes(g_codes, g_scales, o_codes, o_scales, label, flips):
    g_codes, o_codes = np.asarray(g_codes, np.int32), np.asarray(o_codes, np.int32)
    d = np.abs(g_codes - o_codes)
    assert d.max() <= 1, f"{label}: a code differs by {d.max()}"
    flips[0] += int((d > 0).sum())
    flips[1] += d.size
    # a scale is max|x| / 127 of fp32 values that agree with the oracle's within the parity bar
    rel = np.max(np.abs(np.asarray(g_scales, np.float64) - o_scales) / np.maximum(np.abs(o_scales), 1e-30))
    assert rel <= TOL, f"{label}: scales differ by {rel:.2e} relative"
    flips[2] = max(flips[2], rel)


class Ref:
    """The oracle with an int8 cache, teacher-forced on the GPU's tokens."""

    def __init__(self, W, n):
        self.m = oracle.Model(S, W)
        self.c = self.m.new_cache(n)
        self.pos = 0
        self.ties = []

    def step(self, tok, g_lg=None, g_hd=None, g_next=None, label=""):
        lg, hd = self.m.forward_token(int(tok), self.pos, self.c, want_hidden=True)
        self.pos += 1
        if g_lg is not None:
            el, eh = rel_err(g_lg, lg), rel_err(g_hd, hd)
            assert el <= TOL and eh <= TOL, f"{label}: logits {el:.2e} hidden {eh:.2e}"
        if g_next is not None and int(g_next) != oracle.argmax(lg)[0]:
            assert near_tie(lg), f"{label}: token {g_next} != oracle {oracle.argmax(lg)[0]}"
            self.ties.append(label)
        return lg


def test_int8_cache_prefill_and_decode_match_oracle():
    W = weights(S, seed=12)
    cfg = loader.config_from(S)
    assert llmk.decode_path(cfg) == llmk.STEP_PER_OP
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, S.max_seq)
    ref = Ref(W, S.max_seq)
    prompt = synth.prompt(100, S.vocab, stream=71).tolist()
    say("int8 K/V: prefill 100 tokens")
    tok = torch.full((100,), -1, dtype=torch.int32, device="cuda")
    lg = torch.full((S.vocab,), float("nan"), device="cuda")
    hd = torch.full((S.n_layer * S.d,), float("nan"), device="cuda")
    ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, 100))
    assert llmk.prefill(cfg, model, pool, 0, prompt, 0, tok, ws, lg, hd) == llmk.OK
    torch.cuda.synchronize()
    p_tok = host(tok).tolist()
    for i, t in enumerate(prompt):
        ref.step(t, *((host(lg), host(hd).reshape(S.n_layer, S.d)) if i == 99 else (None, None)), p_tok[i],
                 f"prefill {i}")
    dec = loader.Decoder(cfg, model, pool)
    say("int8 K/V: 8 single steps (logits kept), then 60 captured steps")
    fed = [p_tok[-1]]
    for i in range(8):
        lg = torch.empty(S.vocab, device="cuda")
        hd = torch.empty(S.n_layer * S.d, device="cuda")
        assert dec.step(fed[-1], 100 + i, 0, lg, hd) == llmk.OK
        torch.cuda.synchronize()
        nxt = int(host(dec.token_out)[0])
        ref.step(fed[-1], host(lg), host(hd).reshape(S.n_layer, S.d), nxt, f"step {i}")
        fed.append(nxt)
    out = torch.zeros(60, dtype=torch.int32, device="cuda")
    assert dec.steps(fed[-1], 108, 60, out) == llmk.OK
    torch.cuda.synchronize()
    g = host(out).tolist()
    for i in range(60):
        ref.step(fed[-1] if i == 0 else g[i - 1], g_next=g[i], label=f"graph step {i}")
    n = 168
    flips = [0, 0, 0.0]
    for l in range(S.n_layer):
        for w in ("k", "v"):
            cq, cs = pool.read_positions(l, 0, w, 0, n)
            check_codes(host(cq), host(cs), ref.c.codes(l, w)[:n], ref.c.scales(l, w)[:n], f"layer {l} {w}", flips)
    say(f"int8 K/V: {flips[0]} of {flips[1]} codes one step apart, scales within {flips[2]:.1e}; "
        f"near-ties {ref.ties}")
    assert flips[0] * 50 <= flips[1]


def test_int8_cache_batched_rows_match_oracle():
    W = weights(S, seed=12)
    cfg = loader.config_from(S)
    model = loader.upload_model(cfg, W)
    ctxs = [37, 130, 200]
    prefix = synth.kv_prefix_q8(S, max(ctxs), seed=5)
    pool = loader.new_pool(cfg, 3, S.max_seq)
    refs = []
    for r, c in enumerate(ctxs):
        pre = [tuple((kq[:c], ks[:c]) for kq, ks in layer) for layer in prefix]
        loader.fill_prefix(pool, r, pre)
        ref = Ref(W, S.max_seq)
        ref.c.fill_prefix(pre)
        ref.pos = c
        refs.append(ref)
    toks = synth.prompt(3, S.vocab, stream=72).tolist()
    bd = loader.BatchDecoder(cfg, model, pool, 3)
    lg = torch.empty(3 * S.vocab, device="cuda")
    hd = torch.empty(3 * S.n_layer * S.d, device="cuda")
    say("int8 K/V: one batched step over 3 rows (contexts 37, 130, 200)")
    assert bd.step([0, 1, 2], toks, ctxs, lg, hd) == llmk.OK
    torch.cuda.synchronize()
    nxt = host(bd.tokens_out).tolist()
    glg, ghd = host(lg).reshape(3, S.vocab), host(hd).reshape(3, S.n_layer, S.d)
    for r in range(3):
        refs[r].step(toks[r], glg[r], ghd[r], nxt[r], f"row {r}")
    out = torch.zeros(3 * 30, dtype=torch.int32, device="cuda")
    assert bd.steps([0, 1, 2], nxt, [c + 1 for c in ctxs], 30, out) == llmk.OK
    torch.cuda.synchronize()
    g = host(out).reshape(30, 3)
    for j in range(30):
        for r in range(3):
            refs[r].step(nxt[r] if j == 0 else int(g[j - 1, r]), g_next=int(g[j, r]), label=f"graph {j} row {r}")
    flips = [0, 0, 0.0]
    for r, c in enumerate(ctxs):
        for l in range(S.n_layer):
            for w in ("k", "v"):
                cq, cs = pool.read_positions(l, r, w, 0, c + 31)
                check_codes(host(cq), host(cs), refs[r].c.codes(l, w)[:c + 31], refs[r].c.scales(l, w)[:c + 31],
                            f"row {r} layer {l} {w}", flips)
    say(f"int8 K/V batched: {flips[0]} of {flips[1]} codes one step apart, scales within {flips[2]:.1e}; "
        f"near-ties {[x.ties for x in refs]}")
    assert flips[0] * 50 <= flips[1]


def test_int8_paged_pool_forks_and_equals_contiguous():
    W = weights(S, seed=12)
    cfg = loader.config_from(S)
    model = loader.upload_model(cfg, W)
    paged = loader.new_pool(cfg, 2, S.max_seq, block_tokens=64, n_blocks=8)
    flat = loader.new_pool(cfg, 2, S.max_seq)
    prompt = synth.prompt(90, S.vocab, stream=73).tolist()
    res = {}
    for p in (paged, flat):
        tok = torch.full((90,), -1, dtype=torch.int32, device="cuda")
        ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, 90))
        assert llmk.prefill(cfg, model, p, 0, prompt, 0, tok, ws) == llmk.OK
        if p is paged:
            assert llmk.kv_fork(p, 0, 1, 90) == llmk.OK
        else:
            for l in range(S.n_layer):
                for w in ("k", "v"):
                    p.write_positions(l, 1, w, 0, p.read_positions(l, 0, w, 0, 90))
            p.set_len(1, 90)
        dec = loader.Decoder(cfg, model, p)
        outs = []
        for slot, t in ((1, 5), (0, 7), (1, 9)):
            lg = torch.empty(S.vocab, device="cuda")
            assert dec.step(t, int(p.slot_len[slot]), slot, lg) == llmk.OK
            torch.cuda.synchronize()
            outs.append(host(lg))
        res[p is paged] = outs
    for a, b in zip(res[True], res[False]):
        assert np.array_equal(a, b), "paged int8 logits differ from contiguous"
    assert paged.table_h[0, 1] != paged.table_h[1, 1] and paged.table_h[0, 0] == paged.table_h[1, 0]
    for l in range(S.n_layer):
        for w in ("k", "v"):
            for slot in (0, 1):
                a = paged.read_positions(l, slot, w, 0, int(paged.slot_len[slot]))
                b = flat.read_positions(l, slot, w, 0, int(flat.slot_len[slot]))
                assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (l, w, slot)


def test_gqa_attend_over_int8_pool():
    n_layer, n_slots, cap, Hkv, hd, H = 1, 2, 200, 2, 128, 8
    pool = llmk.KVPool(n_layer, n_slots, cap, Hkv, hd, llmk.Q8)
    shape = S.with_(n_layer=1, n_kv=Hkv)
    pre = synth.kv_prefix_q8(shape, 150, seed=8)
    pool.write_positions(0, 1, "k", 0, (dev(pre[0][0][0]).view(150, Hkv, hd), dev(pre[0][0][1]).view(150, Hkv)))
    pool.write_positions(0, 1, "v", 0, (dev(pre[0][1][0]).view(150, Hkv, hd), dev(pre[0][1][1]).view(150, Hkv)))
    pool.set_len(1, 150)
    kv = oracle.q8_rows_value(*pre[0][0]), oracle.q8_rows_value(*pre[0][1])
    for ctx in (1, 64, 65, 150):
        q = synth.normal((H * hd,), 81, ctx, 1.0)
        out = torch.full((H * hd,), float("nan"), device="cuda")
        ws = llmk.workspace(llmk.gqa_attend_workspace_bytes(ctx, H, hd))
        assert llmk.gqa_attend(dev(q), pool, 0, 1, ctx, H, out, ws) == llmk.OK
        torch.cuda.synchronize()
        ref = oracle.attend_f32(q, np.ascontiguousarray(kv[0][:ctx]), np.ascontiguousarray(kv[1][:ctx]), ctx, H, Hkv,
                                hd)
        assert rel_err(host(out), ref) <= TOL, ctx
