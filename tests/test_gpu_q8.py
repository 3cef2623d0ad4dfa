"""int8 weight packs on the GPU (llmk_quantize_q8 and the q8 decode step) against the oracle.

The quantizer's packs equal the oracle's byte for byte (codes are decided in fp32 on both sides). The decode
step over packs quantized on the device, in both forms (one kernel per operation, and the persistent step
kernel streaming the packs, the form the library picks), is checked against the oracle running the decoder the
packs describe
(its own quantization of the same bf16 weights, weights q * s): greedy tokens bit-exact (or a reported
near-tie), logits and per-layer hidden states within the bar. Sizes: a small decoder whose every projection
spans several row blocks with a ragged last one (vocab 1,000, d 256, F 384), the Qwen3-0.6B shape after a
64-position prefix, and the Llama-3-8B shape after its 4,096-position prefix through the launch configuration
the benchmark times (oracle weights rounded once to fp32 there, 2^-24 relative, to bound host memory).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle import quant
from tests.gpu_util import TOL, host, rel_err, say, weights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
llmk = pytest.importorskip("autoregressive_decode_step_amd")
from autoregressive_decode_step_amd import loader  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _matrix(rows, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((rows, K)).astype(np.float32)
    w[:, :K // 2] *= np.float32(1e-3)                         # groups of very different scales
    w[rows // 2, :quant.GROUP] = 0.0                          # an all-zero group
    # a group on the grid of s = 1 with halves: ties to even decide those codes
    w[0, :quant.GROUP] = np.float32(0.5) + rng.integers(-120, 120, quant.GROUP).astype(np.float32)
    w[0, 0] = 127.0
    return w


@pytest.mark.parametrize("rows,K,dtype", [(7, 128, "f32"), (300, 384, "bf16"), (2100, 2048, "bf16"),
                                          (64, 1024, "f32")])
def test_quantize_matches_oracle_bytes(rows, K, dtype):
    w = _matrix(rows, K, seed=rows)
    if dtype == "bf16":
        bits = (w.view(np.uint32) >> 16).astype(np.uint16)    # any bf16 values
        src, ref = loader.to_device(bits), quant.widen(bits)
    else:
        src, ref = loader.to_device(w), w
    nbytes = llmk.q8_pack_bytes(rows, K)
    pack = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device="cuda")
    say(f"quantize {rows} x {K} {dtype}")
    assert llmk.quantize_q8(src, rows, K, pack) == llmk.OK
    torch.cuda.synchronize()
    want = quant.to_pack(*quant.quantize(ref))
    got = host(pack)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:4]}"


def _margin(lg):
    s = np.sort(np.asarray(lg, np.float64))
    return (s[-1] - s[-2]) <= 2 * TOL * np.max(np.abs(s))


def _q8_case(s, n_pre, n_steps, f64, label):
    """Both step forms (one kernel per operation, and the persistent step kernel streaming the packs) against
    the oracle on its own quantization: a free run and teacher-forced steps."""
    say(f"{label}: weights")
    W = weights(s)
    prefix = synth.kv_prefix(s, n_pre, seed=2) if n_pre else None
    first = int(synth.prompt(1, s.vocab, stream=7)[0])

    say(f"{label}: GPU upload and quantization")
    cfgs = {path: loader.config_from(s.with_(w_dtype="q8"), step_path=path)
            for path in (llmk.STEP_PER_OP, llmk.STEP_PERSISTENT)}
    assert llmk.decode_path(loader.config_from(s.with_(w_dtype="q8"))) == llmk.STEP_PERSISTENT   # auto: where it runs
    model = loader.upload_model(cfgs[llmk.STEP_PER_OP], W)

    def new_dec(cfg):
        pool = loader.new_pool(cfg, 1, n_pre + n_steps)
        if prefix:
            loader.fill_prefix(pool, 0, prefix)
        return loader.Decoder(cfg, model, pool)

    gpu_free = {}
    for path, cfg in cfgs.items():
        assert llmk.decode_path(cfg) == path
        toks = torch.zeros(n_steps, dtype=torch.int32, device="cuda")
        assert new_dec(cfg).steps(first, n_pre, n_steps, toks) == llmk.OK
        gpu_free[path] = host(toks).tolist()

    say(f"{label}: oracle on its own quantization")
    m = oracle.Model(s, quant.quantized_weights(W, f64=f64))
    del W
    c = m.new_cache(n_pre + n_steps)
    if prefix:
        c.fill_prefix(prefix)
    t, o_tok, o_lg, o_hid, ties = first, [], [], [], []
    for i in range(n_steps):
        lg, hid = m.forward_token(t, n_pre + i, c, want_hidden=True)
        t = oracle.argmax(lg)[0]
        o_tok.append(t)
        o_lg.append(lg)
        o_hid.append(hid)
        ties.append(_margin(lg))
    say(f"{label}: gpu per-op {gpu_free[llmk.STEP_PER_OP]} persistent {gpu_free[llmk.STEP_PERSISTENT]} "
        f"oracle {o_tok}")

    for path, cfg in cfgs.items():
        name = "per-op" if path == llmk.STEP_PER_OP else "persistent"
        # teacher-forced steps on a fresh pool: logits, hidden states and the token of each step
        dec2 = new_dec(cfg)
        ins = [first] + o_tok[:-1]
        for i, tin in enumerate(ins):
            lg = torch.empty(s.vocab, dtype=torch.float32, device="cuda")
            hid = torch.empty(s.n_layer * s.d, dtype=torch.float32, device="cuda")
            assert dec2.step(tin, n_pre + i, 0, lg, hid) == llmk.OK
            torch.cuda.synchronize()
            el = rel_err(host(lg), o_lg[i])
            eh = rel_err(host(hid).reshape(s.n_layer, s.d), o_hid[i])
            say(f"{label} {name}: step {i}: logits err {el:.2e} hidden err {eh:.2e}")
            assert el <= TOL and eh <= TOL
            g = int(host(dec2.token_out)[0])
            assert g == o_tok[i] or ties[i], f"{label} {name}: step {i}: token {g} != oracle {o_tok[i]}"
        for i, (g, w) in enumerate(zip(gpu_free[path], o_tok)):
            if g != w:
                assert ties[i], f"{label} {name}: free-running step {i}: {g} != {w}"
                break   # after a near-tie the two continuations differ by construction


SMALL = synth.TINY.with_(name="q8 test decoder", vocab=1000, d=256, n_layer=2, n_head=4, n_kv=2, head_dim=64,
                         hidden=384, max_seq=96, w_dtype="bf16")


def test_q8_small_decoder_matches_oracle():
    _q8_case(SMALL, 20, 6, True, "q8 small")


def test_q8_qwen3_shape_matches_oracle():
    _q8_case(synth.Q06, 64, 3, True, "q8 Qwen3-0.6B")


def test_q8_llama8b_full_size_matches_oracle():
    _q8_case(synth.L8B, 4096, 2, False, "q8 8B")
