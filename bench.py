#!/usr/bin/env python3
"""Decode throughput at batch 1 on the Llama-3-8B-shaped decoder, one MI355X.

Workload: bf16 weights N(0, 0.02) (seeded, random init), unit norm gains, RoPE base 5e5, a bf16 K/V
pool whose positions 0..4095 hold seeded N(0, 1) values, then greedy steps from position 4096 with
device-side token feedback (one captured step replayed per token). A step is the whole decode step:
embedding, 32 layers of norm + q|k|v + RoPE + K/V append + attention + o + norm + gate|up + SiLU-gate +
down, final norm, output head and argmax. Inputs are resident in HBM before the timed region.

Prints one JSON line: tokens/s, ms per step, algorithmic HBM GB/s of the whole step, the roofline of
the dominant kernel (the persistent step kernel, or the gate|up GEMV of the per-operation form, timed with
HIP events on the stream it runs on), and the oracle's throughput on the host cores for a bounded sample of
the same workload.

Other workloads (--workload): batched (64 sequences of ragged contexts a step), prefill (a 2,048-token
prompt, Qwen3-0.6B or Llama-3-8B shape), q8 (the batch-1 workload over int8 weight packs), q06 (the
Qwen3-0.6B-shaped decode: 128 greedy steps after a 2,048-token prompt the library prefills), primitives (the
primitive microbenchmark: gemv_t 4096 x 4096 bf16 cold and warm, add_rmsnorm 1 x 4096, RoPE on 32 + 8 heads
over 8,192 positions, argmax over 128,256 logits with planted ties, and the in-place K/V append's cost shape);
--sample T,K,P samples every batch-1 step inside the captured loop; --copy-probe, --sample-probe and
--prefill-probe are short runs for counters and traces.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E, vendor figure
N_PRE = 4096                    # filled context before the first timed step
PMC_FILES = {"gate_up": os.path.join(ROOT, "profiles", "rowdot_gate_up_llama8b_pmc.md"),
             "step": os.path.join(ROOT, "profiles", "step_kernel_llama8b_pmc.md"),
             "gate_up_q8": os.path.join(ROOT, "profiles", "rowdot_q8_gate_up_llama8b_pmc.md"),
             "step_q8": os.path.join(ROOT, "profiles", "step_kernel_q8_llama8b_pmc.md")}
STEP_REPS = 64                  # consecutive steps in the persistent kernel's event timing


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def paged_pool(cfg, n_slots: int, capacity: int, lengths, bt: int):
    """A paged pool whose slot i holds blocks for lengths[i] positions, reserved one block of every slot in
    turn so that each slot's blocks lie scattered through the store (block j of slot i is block
    j * n_slots + i while every slot still needs one)."""
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd import loader
    n_blocks = sum(-(-n // bt) for n in lengths)
    pool = loader.new_pool(cfg, n_slots, capacity, block_tokens=bt, n_blocks=n_blocks)
    for j in range(max(-(-n // bt) for n in lengths)):
        for i, n in enumerate(lengths):
            if j * bt < n:
                st = llmk.kv_reserve(pool, i, j * bt, min(n, (j + 1) * bt))
                if st != llmk.OK:
                    raise RuntimeError(f"kv_reserve: {st} {llmk.status_name(st)}")
    return pool


def q8_pack_bytes(rows: int, cols: int) -> int:
    """Bytes of an int8 weight pack: a code per weight and an fp32 scale per 128 inputs of a row."""
    return rows * cols + 4 * rows * (cols // 128)


def step_bytes(s, ctx: int, q8: bool = False) -> int:
    """Algorithmic HBM bytes of one decode step attending `ctx` positions: every weight once, the
    embedding row, the gains, the RoPE table row, the K/V of the attended context, the appended K/V,
    and the logits written once. q8: the projections and the head are int8 packs (embedding bf16)."""
    wsz = 2 if s.w_dtype == "bf16" else 4
    kvsz = 2 if s.kv_dtype == "bf16" else 4
    d, qd, kvd, F, V, L = s.d, s.n_head * s.head_dim, s.n_kv * s.head_dim, s.hidden, s.vocab, s.n_layer
    if q8:
        pb = q8_pack_bytes
        weights = L * (pb(qd, d) + 2 * pb(kvd, d) + pb(d, qd) + 2 * pb(F, d) + pb(d, F)) + pb(V, d) + d * 2
    else:
        weights = L * (d * qd + 2 * d * kvd + qd * d + 3 * d * F) * wsz + V * d * wsz + d * wsz
    gains = (2 * L + 1) * d * 4
    rope = s.head_dim * 4
    kv = L * ctx * kvd * 2 * kvsz + L * kvd * 2 * kvsz
    logits = V * 4
    return weights + gains + rope + kv + logits


def gate_up_bytes(s, q8: bool = False) -> int:
    """Algorithmic bytes of one gate|up launch: both weight matrices, the input row, its gain, u written."""
    wsz = 2 if s.w_dtype == "bf16" else 4
    w = 2 * q8_pack_bytes(s.hidden, s.d) if q8 else 2 * s.d * s.hidden * wsz
    return w + 2 * s.d * 4 + s.hidden * 4


KERNEL_SOURCES = {"gate_up": ("rowdot.hip", "common.h", "kernels.h"),
                  "step": ("step.hip", "attn_block.h", "common.h", "kernels.h"),
                  "gate_up_q8": ("q8.hip", "q8.h", "common.h", "kernels.h"),
                  "step_q8": ("step.hip", "attn_block.h", "common.h", "kernels.h")}


def kernel_source_sha(which: str = "gate_up") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        with open(os.path.join(ROOT, "autoregressive_decode_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(which: str):
    """HBM bytes per launch of the dominant kernel (`which`: a PMC_FILES key) from the committed counter
    summary ("key: value" lines), if its counters were taken on the current kernel source; None otherwise."""
    rec = {}
    try:
        with open(PMC_FILES[which]) as f:
            for line in f:
                k, sep, v = line.partition(":")
                if sep:
                    rec[k.strip()] = v.strip()
    except OSError:
        return None
    if rec.get("source_sha") != kernel_source_sha(which):
        return None
    try:
        return int(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_probe(mib: int) -> int:
    """A plain device-to-device copy of `mib` MiB, run 4 times: reads and writes that many bytes per launch.
    Run under the same counters as the decode step, it gives the scale between what FETCH_SIZE / WRITE_SIZE
    report and bytes actually moved."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(4):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_per_launch": n * 4, "launches": 4}), flush=True)
    return 0


def sample_probe(rows: int, reps: int = 50) -> int:
    """Only the sampling exit: llmk_sample over `rows` vocabulary rows (128,256 logits, N(0, 3)) at
    temperature 0.8, top-k 50, top-p 0.95, timed with HIP events over `reps` launches."""
    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd.loader import to_device
    n = synth.L8B.vocab
    logits = to_device(synth.normal((rows, n), 600, 0, 3.0).ravel(), "cuda")
    u = to_device(synth.draws((rows,), 601, 0), "cuda")
    tok = torch.empty(rows, dtype=torch.int32, device="cuda")
    ws = llmk.workspace(llmk.sample_workspace_bytes(rows, n, 0.8, 50))
    stream = torch.cuda.current_stream()

    def once():
        st = llmk.sample(logits, rows, n, 0.8, 50, 0.95, u, tok, ws)
        if st != llmk.OK:
            raise RuntimeError(f"llmk_sample: {st} {llmk.status_name(st)}")

    for _ in range(5):
        once()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        once()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    alg = rows * n * 4
    print(json.dumps({"sample_probe": {"rows": rows, "n": n, "temperature": 0.8, "top_k": 50, "top_p": 0.95,
                                       "us_per_launch": round(us, 2), "algorithmic_bytes": alg,
                                       "achieved_GBps": round(alg / us / 1e3, 1)}}), flush=True)
    return 0


def prefill_probe(shape: str, n: int = 2048, reps: int = 3) -> int:
    """Only prefill: an n-token seeded prompt into an empty slot of the named shape (q06: Qwen3-0.6B, the
    2,048-token prefix workload; l8b: Llama-3-8B), timed over `reps` calls after one warm-up call."""
    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd import loader
    s = {"q06": synth.Q06, "l8b": synth.L8B}[shape]
    log(f"generating {s.name} weights")
    W = synth.model(s, seed=0)
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    del W
    pool = loader.new_pool(cfg, 1, n + 8)
    tokens = synth.prompt(n, s.vocab, stream=23).tolist()
    ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, n))
    out = torch.zeros(n, dtype=torch.int32, device="cuda")

    def once():
        pool.slot_len[0] = 0
        st = llmk.prefill(cfg, model, pool, 0, tokens, 0, out, ws)
        if st != llmk.OK:
            raise RuntimeError(f"llmk_prefill: {st} {llmk.status_name(st)}")

    once()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        once()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / reps
    print(json.dumps({"prefill_probe": {"shape": s.name, "prompt_tokens": n, "ms_per_prompt": round(ms, 2),
                                        "tokens_per_s": round(n / ms * 1e3, 1)}}), flush=True)
    return 0


PREFILL_TOKENS = 2048
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 matrix-core peak


def prefill_flops(s, n: int, pos0: int = 0) -> dict:
    """Algorithmic flops of an n-token prefill from position pos0: the projections (2 flops per weight per row)
    and causal attention (q.k and p.v over each row's visible positions, 4 hd flops per position and head)."""
    d, qd, kvd, F, L = s.d, s.n_head * s.head_dim, s.n_kv * s.head_dim, s.hidden, s.n_layer
    proj = 2 * n * L * (d * (qd + 2 * kvd) + qd * d + 2 * d * F + F * d)
    attn = 4 * s.head_dim * s.n_head * L * sum(pos0 + i + 1 for i in range(n))
    head = 2 * n * s.vocab * d
    return {"projections": proj, "attention": attn, "head": head}


def run_prefill(args) -> int:
    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd import loader
    s = {"q06": synth.Q06, "l8b": synth.L8B}[args.prefill_shape]
    n = PREFILL_TOKENS
    steps = args.steps if args.steps != 256 else 8
    t_start = time.time()
    log(f"generating {s.name} weights")
    W = synth.model(s, seed=0)
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, n + 8)
    tokens = synth.prompt(n, s.vocab, stream=23).tolist()
    ws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, n))
    out = torch.zeros(n, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    log(f"resident in HBM after {time.time() - t_start:.1f} s")

    def once():
        pool.slot_len[0] = 0
        st = llmk.prefill(cfg, model, pool, 0, tokens, 0, out, ws)
        if st != llmk.OK:
            raise RuntimeError(f"llmk_prefill: {st} {llmk.status_name(st)}")

    for _ in range(max(args.warmup, 1)):
        once()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        once()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = elapsed * 1e3 / steps
    pool.slot_len[0] = 0
    st, phase_ms = llmk.prefill_profiled(cfg, model, pool, 0, tokens, 0, out, ws)
    if st != llmk.OK:
        raise RuntimeError(f"llmk_prefill_profiled: {st} {llmk.status_name(st)}")
    gpu_tokens = out.cpu().tolist()
    fl = prefill_flops(s, n)
    log(f"timed {steps} prompts of {n} tokens: {ms:.2f} ms each, {n / ms * 1e3:.0f} tokens/s; phases (ms) "
        + ", ".join(f"{k} {v:.2f}" for k, v in phase_ms.items()))
    dom = max(("projections", "attention"), key=lambda k: phase_ms[k])
    tflops = fl[dom] / (phase_ms[dom] * 1e-3) / 1e12
    result = {
        "metric": f"prefill tokens/s ({n}-token prompt)",
        "value": n / ms * 1e3,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": max(args.warmup, 1),
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{s.name} prefill of a {n}-token seeded prompt into an empty slot, chunks of 256 "
                               "rows, projections and attention on bf16 matrix cores (activations as bf16 hi + lo)",
                   "prompt_tokens": n, "chunk_rows": 256, "weights": s.w_dtype, "kv": s.kv_dtype,
                   "accumulation": "f32"},
        "phase_ms": phase_ms,
        "roofline": {"bound": "mfma", "kernel": "prefill " + dom + (" (pgemm_kernel + epilogue)" if dom == "projections"
                                                                    else " (rope_append + fattn_kernel + merge)"),
                     "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None,
                     "flops_per_prompt": fl[dom], "ms_per_prompt": phase_ms[dom],
                     "note": "algorithmic flops; the bf16 hi + lo activations make the matrix cores execute twice "
                             "(three times against fp32 K/V) as many"},
    }
    if not args.no_cpu_baseline:
        import oracle
        k = args.cpu_prefill_tokens
        log(f"oracle baseline: the first {k} prompt tokens, one at a time, on the host cores")
        m = oracle.Model(s, W)
        c = m.new_cache(k)
        otoks = []
        tc0 = time.perf_counter()
        for i in range(k):
            lg, _ = m.forward_token(tokens[i], i, c)
            otoks.append(oracle.argmax(lg)[0])
        tc = time.perf_counter() - tc0
        result["cpu_baseline"] = {"value": k / tc, "unit": "tokens/s", "cores": oracle.lib().orc_num_threads(),
                                  "kind": "oracle",
                                  "sample": f"the first {k} tokens of the same prompt, one decode step each (fp64, "
                                            f"OpenMP)",
                                  "tokens_agree_with_gpu": otoks == gpu_tokens[:k]}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    log(f"total {time.time() - t_start:.1f} s")
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed greedy decode steps")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--kernel-reps", type=int, default=4,
                    help="times each kernel class's per-layer launches are replayed for its HIP-event timing")
    ap.add_argument("--cpu-steps", type=int, default=20, help="oracle steps in the CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", choices=("batch1", "batched", "prefill", "q8", "q06", "primitives"), default="batch1",
                    help="batch1: the 8B-shaped single-sequence step (default); batched: 64 ragged sequences per step; "
                         "prefill: a 2,048-token prompt (steps = prompts, 8 by default); q06: Qwen3-0.6B-shaped decode "
                         "after a 2,048-token prompt; primitives: the primitive microbenchmark")
    ap.add_argument("--prefill-shape", choices=("q06", "l8b"), default="q06",
                    help="the prefill workload's shape: Qwen3-0.6B (the 2,048-token prefix workload) or Llama-3-8B")
    ap.add_argument("--cpu-prefill-tokens", type=int, default=24, help="oracle tokens in the prefill CPU baseline")
    ap.add_argument("--sample", type=lambda v: tuple(float(x) for x in v.split(",")), default=None,
                    metavar="T,K,P", help="batch-1 workloads: sample every step (temperature, top-k, top-p) inside "
                                         "the captured loop instead of taking the greedy token")
    ap.add_argument("--kv", choices=("bf16", "q8"), default="bf16",
                    help="batched: the K/V cache dtype (q8: int8 rows with an fp32 scale per position and head)")
    ap.add_argument("--paged", type=int, default=0, metavar="BLOCK_TOKENS",
                    help="batch1 / batched: hold the K/V in a paged pool of blocks of this many positions")
    ap.add_argument("--step-path", choices=("auto", "per-op", "persistent"), default="auto",
                    help="the decode step's form: the library's choice (default), one kernel per operation, or "
                         "the persistent one-kernel step")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    ap.add_argument("--prefill-probe", choices=("q06", "l8b"), default=None,
                    help="only time a 2,048-token prefill of the named shape and exit")
    ap.add_argument("--sample-probe", type=int, default=0, metavar="ROWS",
                    help="only time the sampling exit over ROWS vocabulary rows and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: the "
              f"decode step here is single-GPU by design", file=sys.stderr)
        return 2

    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd import loader

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 3
    if args.copy_probe > 0:
        return copy_probe(args.copy_probe)
    if args.prefill_probe:
        return prefill_probe(args.prefill_probe)
    if args.sample_probe > 0:
        return sample_probe(args.sample_probe)
    if args.workload == "batched":
        return run_batched(args)
    if args.workload == "prefill":
        return run_prefill(args)
    if args.workload == "q06":
        return run_q06(args)
    if args.workload == "primitives":
        return run_primitives(args)

    s = synth.L8B
    q8 = args.workload == "q8"
    max_steps_per_call = s.max_seq - N_PRE
    t_start = time.time()
    log(f"generating {s.name} weights")
    W = synth.model(s, seed=0)
    prefix = synth.kv_prefix(s, N_PRE, seed=2)
    first = int(synth.prompt(1, s.vocab, stream=7)[0])
    log(f"generated in {time.time() - t_start:.1f} s; uploading")
    path_arg = {"auto": llmk.STEP_AUTO, "per-op": llmk.STEP_PER_OP, "persistent": llmk.STEP_PERSISTENT}[args.step_path]
    cfg = loader.config_from(s.with_(w_dtype="q8") if q8 else s, step_path=path_arg)
    path = llmk.decode_path(cfg)
    if path not in (llmk.STEP_PER_OP, llmk.STEP_PERSISTENT):
        raise RuntimeError(f"decode_path: {path} {llmk.status_name(path)}")
    persistent = path == llmk.STEP_PERSISTENT
    model = loader.upload_model(cfg, W)
    if args.paged:
        # slot 0 runs; slot 1 only interleaves its blocks with slot 0's
        pool = paged_pool(cfg, 2, s.max_seq, [s.max_seq, s.max_seq], args.paged)
    else:
        pool = loader.new_pool(cfg, 1, s.max_seq)
    loader.fill_prefix(pool, 0, prefix)
    dec = loader.Decoder(cfg, model, pool)
    torch.cuda.synchronize()
    log(f"resident in HBM after {time.time() - t_start:.1f} s; step form: {'persistent' if persistent else 'per-op'}")

    if args.sample:
        s_t, s_k, s_p = args.sample[0], int(args.sample[1]), args.sample[2]
        draws = torch.from_numpy(synth.draws((max_steps_per_call,), seed=5, stream=31)).cuda()
        sample_ws = llmk.workspace(max(llmk.sample_workspace_bytes(1, s.vocab, s_t, s_k), 16))

    def run(n: int, out) -> None:
        done = 0
        while done < n:
            k = min(max_steps_per_call, n - done)
            pool.slot_len[0] = N_PRE
            if args.sample:
                st = llmk.decode_steps_sampled(cfg, model, pool, 0, first, N_PRE, k, s_t, s_k, s_p, draws[:k],
                                               out[done:done + k], dec.ws, sample_ws)
            else:
                st = dec.steps(first, N_PRE, k, out[done:done + k])
            if st != llmk.OK:
                raise RuntimeError(f"decode_steps: {st} {llmk.status_name(st)}")
            done += k

    # warm-up (not timed)
    warm = torch.zeros(max(args.warmup, 1), dtype=torch.int32, device="cuda")
    if args.warmup > 0:
        run(args.warmup, warm)
    torch.cuda.synchronize()

    # timed region
    toks = torch.zeros(args.steps, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.steps, toks)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    elapsed = t1 - t0
    ms_per_step = elapsed * 1e3 / args.steps
    ctxs = [N_PRE + 1 + (i % max_steps_per_call) for i in range(args.steps)]
    total_bytes = sum(step_bytes(s, c, q8) for c in ctxs)
    step_gbps = total_bytes / elapsed / 1e9
    tokens = toks.cpu().numpy().tolist()
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step, {step_gbps:.0f} GB/s algorithmic")

    # kernel timing with HIP events on the stream the kernels run on
    pool.slot_len[0] = N_PRE
    avg_ms = {}
    if persistent:
        # the persistent form is one kernel per step: STEP_REPS consecutive steps replayed back to back
        st, ms = llmk.decode_kernel_time(cfg, model, pool, 0, first, N_PRE, llmk.STEP_KERNEL, STEP_REPS,
                                         dec.token_out, dec.ws)
        if st != llmk.OK:
            raise RuntimeError(f"decode_kernel_time(step): {st} {llmk.status_name(st)}")
        pool.slot_len[0] = N_PRE
        avg_ms["step"] = ms
        k_bytes = sum(step_bytes(s, N_PRE + 1 + i, q8) for i in range(STEP_REPS)) / STEP_REPS
        k_name = "persistent decode step (step_kernel, the whole step in one launch)"
        kernel_sum_ms = ms
    else:
        # each class's launches (every layer, several times over) replayed back to back in one graph
        for k, n in enumerate(llmk.KERNEL_CLASSES):
            st, ms = llmk.decode_kernel_time(cfg, model, pool, 0, first, N_PRE, k, args.kernel_reps, dec.token_out,
                                             dec.ws)
            if st != llmk.OK:
                raise RuntimeError(f"decode_kernel_time({n}): {st} {llmk.status_name(st)}")
            avg_ms[n] = ms
            pool.slot_len[0] = N_PRE
        k_bytes = gate_up_bytes(s, q8)
        ms = avg_ms["gate_up"]
        k_name = ("gate|up row-dot GEMV over int8 packs (rowdot_q8_kernel, GATEUP epilogue)" if q8 else
                  "gate|up row-dot GEMV (rowdot_kernel, GATEUP epilogue)")
        kernel_sum_ms = sum(avg_ms[n] for n in llmk.KERNEL_CLASSES[:5]) * s.n_layer + avg_ms["head"]
    k_gbps = k_bytes / (ms * 1e-3) / 1e9
    log("avg kernel us: " + ", ".join(f"{n} {v * 1e3:.1f}" for n, v in avg_ms.items()))

    result = {
        "metric": ("decode tokens/s at batch 1 (8B-shaped, int8 weight packs) + achieved HBM GB/s vs peak" if q8
                   else "decode tokens/s at batch 1 (8B-shaped) + achieved HBM GB/s vs peak"),
        "value": args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": ("llama-3-8b-shaped greedy decode, batch 1, int8 weight packs (projections and head; "
                                "fp32 scale per 128 inputs), bf16 embedding and K/V, context 4096" if q8 else
                                "llama-3-8b-shaped greedy decode, batch 1, bf16 weights and K/V, context 4096"),
                   "vocab": s.vocab, "d": s.d, "n_layer": s.n_layer, "n_head": s.n_head, "n_kv": s.n_kv,
                   "head_dim": s.head_dim, "hidden": s.hidden, "batch": 1, "context_start": N_PRE,
                   "weights": "q8" if q8 else "bf16", "kv": "bf16", "accumulation": "f32",
                   "kv_pool": (f"paged, {args.paged}-position blocks interleaved with another slot's" if args.paged
                               else "contiguous slot")},
        "step_hbm_gbps": step_gbps,
        "step_frac_of_peak": step_gbps / PEAK_HBM_GBPS,
        "step_bytes_mean": total_bytes / args.steps,
        "step_form": "persistent" if persistent else "per-op",
        "roofline": {"bound": "hbm", "kernel": k_name,
                     "achieved": k_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": k_gbps / PEAK_HBM_GBPS,
                     "traffic": traffic_from_profiles(("step_q8" if q8 else "step") if persistent else
                                                      ("gate_up_q8" if q8 else "gate_up")),
                     "bytes_per_launch": k_bytes, "avg_launch_us": ms * 1e3},
        "kernels_avg_us": {n: v * 1e3 for n, v in avg_ms.items()},
        "kernel_sum_ms_per_step": kernel_sum_ms,
        "first_tokens": tokens[:8],
    }
    if args.sample:
        result["config"]["sampling"] = {"temperature": s_t, "top_k": s_k, "top_p": s_p,
                                        "draws": "seeded uniforms, one per step"}

    if args.sample and not args.no_cpu_baseline:
        log("the CPU baseline runs the greedy workload; skipped for a sampled run")
    if not args.no_cpu_baseline and not args.sample:
        import oracle
        n = args.cpu_steps
        log(f"oracle baseline: {n} steps on the host cores")
        if q8:
            from oracle import quant
            log("oracle: the decoder the int8 packs describe (fp32 copies of q * s)")
            Wq = quant.quantized_weights(W, f64=False)
            m = oracle.Model(s, Wq)
        else:
            m = oracle.Model(s, W)
        c = m.new_cache(N_PRE + n)
        c.fill_prefix(prefix)
        t = first
        otoks = []
        tc0 = time.perf_counter()
        for i in range(n):
            lg, _ = m.forward_token(t, N_PRE + i, c)
            t = oracle.argmax(lg)[0]
            otoks.append(t)
        tc = time.perf_counter() - tc0
        result["cpu_baseline"] = {"value": n / tc, "unit": "tokens/s", "cores": oracle.lib().orc_num_threads(),
                                  "kind": "oracle",
                                  "sample": f"{n} greedy decode steps of the same workload at positions "
                                            f"{N_PRE}..{N_PRE + n - 1} (fp64, OpenMP"
                                            + (", weights q * s of the oracle's own quantization)" if q8 else ")"),
                                  "tokens_agree_with_gpu": otoks == tokens[:n]}
        log(f"oracle: {tc / n:.2f} s/step, tokens {otoks} vs gpu {tokens[:n]}")
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    log(f"total {time.time() - t_start:.1f} s")
    return 0


Q06_PROMPT = 2048               # tokens the Qwen3-0.6B-shaped workload prefills before decoding
Q06_STEPS = 128                 # greedy steps it decodes (positions 2,048..2,175)


def run_q06(args) -> int:
    """The Qwen3-0.6B-shaped decode: a seeded 2,048-token prompt through the library's prefill, then greedy
    steps at positions 2,048..2,175 (one captured step replayed per token), timed like the 8B workload."""
    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd import loader
    s = synth.Q06
    steps = args.steps if args.steps != 256 else Q06_STEPS
    if steps > Q06_STEPS or args.warmup > Q06_STEPS:
        print(f"the q06 workload has room for {Q06_STEPS} steps per run", file=sys.stderr)
        return 2
    t_start = time.time()
    log(f"generating {s.name} weights")
    W = synth.model(s, seed=0)
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    pool = loader.new_pool(cfg, 1, s.max_seq)
    prompt = synth.prompt(Q06_PROMPT, s.vocab, stream=23).tolist()
    pws = llmk.workspace(llmk.prefill_workspace_bytes(cfg, Q06_PROMPT))
    ptoks = torch.zeros(Q06_PROMPT, dtype=torch.int32, device="cuda")
    st = llmk.prefill(cfg, model, pool, 0, prompt, 0, ptoks, pws)
    if st != llmk.OK:
        raise RuntimeError(f"llmk_prefill: {st} {llmk.status_name(st)}")
    del pws
    first = int(ptoks[-1].item())
    dec = loader.Decoder(cfg, model, pool)
    persistent = llmk.decode_path(cfg) == llmk.STEP_PERSISTENT
    torch.cuda.synchronize()
    log(f"prompt prefilled, resident in HBM after {time.time() - t_start:.1f} s; step form: "
        f"{'persistent' if persistent else 'per-op'}")

    def run(n, out):
        pool.slot_len[0] = Q06_PROMPT
        st = dec.steps(first, Q06_PROMPT, n, out)
        if st != llmk.OK:
            raise RuntimeError(f"decode_steps: {st} {llmk.status_name(st)}")

    if args.warmup > 0:
        run(args.warmup, torch.zeros(args.warmup, dtype=torch.int32, device="cuda"))
    toks = torch.zeros(steps, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps, toks)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    total_bytes = sum(step_bytes(s, Q06_PROMPT + 1 + i) for i in range(steps))
    gbps = total_bytes / elapsed / 1e9
    log(f"timed {steps} steps: {ms_per_step:.3f} ms/step, {steps / elapsed:.0f} tokens/s, {gbps:.0f} GB/s algorithmic")
    pool.slot_len[0] = Q06_PROMPT
    reps = min(STEP_REPS, Q06_STEPS)
    kind = llmk.STEP_KERNEL if persistent else llmk.KERNEL_CLASSES.index("gate_up")
    st, kms = llmk.decode_kernel_time(cfg, model, pool, 0, first, Q06_PROMPT, kind, reps if persistent else 4,
                                      dec.token_out, dec.ws)
    if st != llmk.OK:
        raise RuntimeError(f"decode_kernel_time: {st} {llmk.status_name(st)}")
    k_bytes = (sum(step_bytes(s, Q06_PROMPT + 1 + i) for i in range(reps)) / reps if persistent
               else gate_up_bytes(s))
    k_gbps = k_bytes / (kms * 1e-3) / 1e9
    result = {
        "metric": "decode tokens/s at batch 1 (Qwen3-0.6B-shaped, after a 2,048-token prompt) + achieved HBM GB/s",
        "value": steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "qwen3-0.6b-shaped greedy decode, batch 1, a seeded 2,048-token prompt prefilled by "
                               "the library, then steps at positions 2,048..2,175; bf16 weights, fp32 K/V",
                   "vocab": s.vocab, "d": s.d, "n_layer": s.n_layer, "n_head": s.n_head, "n_kv": s.n_kv,
                   "head_dim": s.head_dim, "hidden": s.hidden, "batch": 1, "context_start": Q06_PROMPT,
                   "weights": "bf16", "kv": "f32", "accumulation": "f32"},
        "step_hbm_gbps": gbps,
        "step_frac_of_peak": gbps / PEAK_HBM_GBPS,
        "step_bytes_mean": total_bytes / steps,
        "step_form": "persistent" if persistent else "per-op",
        "roofline": {"bound": "hbm",
                     "kernel": ("persistent decode step (step_kernel)" if persistent else
                                "gate|up row-dot GEMV (rowdot_kernel, GATEUP epilogue)"),
                     "achieved": k_gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": k_gbps / PEAK_HBM_GBPS,
                     "traffic": None, "bytes_per_launch": k_bytes, "avg_launch_us": kms * 1e3},
        "first_tokens": toks[:8].cpu().tolist(),
    }
    if not args.no_cpu_baseline:
        import oracle
        n = args.cpu_steps
        log(f"oracle baseline: {n} steps over a 2,048-position cache on the host cores")
        m = oracle.Model(s, W)
        c = m.new_cache(Q06_PROMPT + n)
        c.fill_prefix(synth.kv_prefix(s, Q06_PROMPT, seed=2))
        t = first
        tc0 = time.perf_counter()
        for i in range(n):
            lg, _ = m.forward_token(t, Q06_PROMPT + i, c)
            t = oracle.argmax(lg)[0]
        tc = time.perf_counter() - tc0
        result["cpu_baseline"] = {"value": n / tc, "unit": "tokens/s", "cores": oracle.lib().orc_num_threads(),
                                  "kind": "oracle",
                                  "sample": f"{n} greedy decode steps at positions {Q06_PROMPT}..{Q06_PROMPT + n - 1} "
                                            "over a 2,048-position cache of seeded K/V (the same sizes and work as the "
                                            "timed steps; the prompt itself is not run through the oracle here, so the "
                                            "tokens are not compared) (fp64, OpenMP)"}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    log(f"total {time.time() - t_start:.1f} s")
    return 0


def run_primitives(args) -> int:
    """The primitive microbenchmark, each primitive through the C ABI on seeded inputs: many calls captured in a
    graph on the stream the binding launches on and replayed between HIP events (device time per call), and each
    primitive of the oracle timed on the host cores for the same inputs."""
    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd.loader import to_device
    stream = torch.cuda.Stream()      # default priority; graphs are captured on it and replayed on it
    torch.cuda.set_stream(stream)

    def timed(fn, reps):
        """Device time per call: `reps` calls captured once into a graph, the graph replayed between two events
        (so host launch costs are not counted), after an eager warm-up."""
        for _ in range(3):
            fn(0)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps   # us per call

    def check(st, what):
        if st != llmk.OK:
            raise RuntimeError(f"{what}: {st} {llmk.status_name(st)}")

    out = {}
    # gemv_t: y = A^T x, A 4096 x 4096 bf16 N(0, 0.02), x fp32 N(0, 1); cold = 16 rotated copies (537 MB, past
    # the 256 MB of last-level cache), warm = one copy
    m = n = 4096
    a_np = synth.normal((m, n), 10, 0, 0.02, "bf16")
    x_np = synth.normal((m,), 10, 1, 1.0)
    copies = [to_device(a_np) for _ in range(16)]
    x = to_device(x_np)
    y = torch.empty(n, dtype=torch.float32, device="cuda")
    ws = llmk.workspace(llmk.gemv_t_workspace_bytes(m, n, llmk.BF16))
    gb = m * n * 2 + m * 4 + n * 4
    check(llmk.gemv_t(copies[0], x, y, m, n, ws), "gemv_t")
    torch.cuda.synchronize()
    y_eager = y.clone()
    cold = timed(lambda i: check(llmk.gemv_t(copies[i % 16], x, y, m, n, ws), "gemv_t"), 160)
    warm = timed(lambda i: check(llmk.gemv_t(copies[0], x, y, m, n, ws), "gemv_t"), 160)
    if not torch.equal(y, y_eager):   # every copy holds the same A: a replayed call gives the eager result, bit for bit
        raise RuntimeError("gemv_t: a replayed call differs from the eager one")
    out["gemv_t_4096x4096_bf16"] = {"algorithmic_bytes": gb, "us_cold": cold, "GBps_cold": gb / cold / 1e3,
                                    "frac_cold": gb / cold / 1e3 / PEAK_HBM_GBPS, "us_warm": warm,
                                    "GBps_warm": gb / warm / 1e3, "cold_copies": 16}
    del copies
    # add_rmsnorm 1 x 4096: residual and x N(0, 1), gain 1 + N(0, 0.1), eps 1e-5
    r_np = synth.normal((4096,), 11, 0, 1.0)
    xr_np = synth.normal((4096,), 11, 1, 1.0)
    g_np = synth.normal((4096,), 11, 2, 0.1, mean=1.0)
    r, xr, g, h = to_device(r_np), to_device(xr_np), to_device(g_np), torch.empty(4096, dtype=torch.float32,
                                                                                     device="cuda")
    us = timed(lambda i: check(llmk.add_rmsnorm(r, xr, g, h, 1, 4096, 1e-5), "add_rmsnorm"), 500)
    out["add_rmsnorm_1x4096"] = {"algorithmic_bytes": 81920, "us": us, "GBps": 81920 / us / 1e3}
    # RoPE: q [8192][32][128], k [8192][8][128] fp32 N(0, 1), row r at position r, base 1e4 and 5e5; one position
    # alone (its latency) and the whole sweep in one launch
    rows, nq, nk, hd = 8192, 32, 8, 128
    q_np = synth.normal((rows * nq * hd,), 12, 0, 1.0)
    k_np = synth.normal((rows * nk * hd,), 12, 1, 1.0)
    qd, kd = to_device(q_np), to_device(k_np)
    pos = torch.arange(rows, dtype=torch.int32, device="cuda")
    rope = {}
    for base in (1e4, 5e5):
        tab = torch.empty(rows * hd, dtype=torch.float32, device="cuda")
        check(llmk.rope_table_init(tab, rows, hd, base), "rope_table_init")
        sweep = timed(lambda i: check(llmk.rope(qd, kd, rows, nq, nk, hd, pos, tab, rows, 0), "rope"), 50)
        one = timed(lambda i: check(llmk.rope(qd[:nq * hd], kd[:nk * hd], 1, nq, nk, hd, pos[4095:4096], tab, rows, 0),
                                    "rope"), 500)
        b = rows * 41472
        rope[f"base_{base:g}"] = {"us_one_position": one, "us_sweep_8192": sweep, "sweep_bytes": b,
                                  "GBps_sweep": b / sweep / 1e3}
    out["rope_32q_8k_hd128"] = rope
    # argmax over 128,256 fp32 N(0, 3) with planted exact ties across a workgroup slice boundary
    V = 128256
    lg_np = synth.normal((V,), 13, 0, 3.0)
    mx = float(lg_np.max()) + 0.5
    lg_np[[2003, 2004, 90000]] = mx
    lg = to_device(lg_np)
    tok = torch.empty(1, dtype=torch.int32, device="cuda")
    val = torch.empty(1, dtype=torch.float32, device="cuda")
    aws = llmk.workspace(llmk.argmax_workspace_bytes(1, V))
    us = timed(lambda i: check(llmk.argmax(lg, 1, V, tok, val, aws), "argmax"), 500)
    out["argmax_128256"] = {"algorithmic_bytes": V * 4, "us": us, "GBps": V * 4 / us / 1e3,
                            "token": int(tok.item()), "planted_tie_lowest_index": 2003}
    # the in-place K/V append's cost shape: one decode token's K row (8 heads x 128 = 1,024 elements) appended to a
    # bf16 cache holding 2,048 and 133,120 elements; per-element time growth (the gate is 3x)
    cache = torch.zeros(140000, dtype=torch.bfloat16, device="cuda")
    newv = to_device(synth.normal((1024,), 14, 0, 1.0))
    per = {}
    for filled in (2048, 133120):
        us = timed(lambda i: check(llmk.kv_append_flat(cache, filled, filled, newv)[0], "kv_append_flat"), 500)
        per[filled] = us / 1024
    out["kv_append_cost_shape"] = {"n_new": 1024, "us_per_element_at_2048": per[2048],
                                   "us_per_element_at_133120": per[133120], "growth": per[133120] / per[2048],
                                   "gate": 3.0}
    log("primitives: " + json.dumps(out))
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        log("oracle baseline: each primitive on the host cores")
        c = {}
        t0 = time.perf_counter()
        for _ in range(5):
            oracle.gemv_t_f32(a_np, x_np)
        c["gemv_t_4096x4096_bf16_us"] = (time.perf_counter() - t0) / 5 * 1e6
        t0 = time.perf_counter()
        for _ in range(200):
            oracle.add_rmsnorm_f32(r_np, xr_np, g_np, 1, 4096, 1e-5)
        c["add_rmsnorm_1x4096_us"] = (time.perf_counter() - t0) / 200 * 1e6
        t0 = time.perf_counter()
        oracle.rope_f32(q_np, k_np, rows, nq, nk, hd, 0, 1e4, 0)
        c["rope_sweep_8192_us"] = (time.perf_counter() - t0) * 1e6
        t0 = time.perf_counter()
        for _ in range(20):
            o_tok, _ = oracle.argmax(lg_np)
        c["argmax_128256_us"] = (time.perf_counter() - t0) / 20 * 1e6
        c["argmax_token"] = o_tok
        cpu = {"value": gb / c["gemv_t_4096x4096_bf16_us"] / 1e3, "unit": "GB/s", "cores": oracle.lib().orc_num_threads(),
               "kind": "oracle",
               "sample": "each primitive of the oracle on the same inputs (fp64): gemv_t 5 calls, add_rmsnorm 200, "
                         "the RoPE sweep once, argmax 20; value = the oracle gemv_t's algorithmic GB/s",
               "per_primitive": c}
    g = out["gemv_t_4096x4096_bf16"]
    result = {
        "metric": "primitive microbench: gemv_t 4096x4096 bf16 GB/s (cold) with add_rmsnorm, RoPE and argmax latencies",
        "value": g["GBps_cold"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": 160,
        "warmup": 3,
        "ms_per_step": g["us_cold"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "primitive microbench: gemv_t A 4096x4096 bf16 N(0,0.02), x fp32 N(0,1) (16 rotated "
                               "copies of A for the cold figure); add_rmsnorm 1x4096; RoPE on 32 q + 8 k heads at hd 128, "
                               "positions 0..8191; argmax over 128,256 fp32 N(0,3) with planted exact ties; in-place "
                               "K/V append cost shape"},
        "primitives": out,
        "roofline": {"bound": "hbm", "kernel": "gemv_t (gemv_t_kernel, split-K over A[in][out]), cold",
                     "achieved": g["GBps_cold"], "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": g["frac_cold"],
                     "traffic": None, "bytes_per_launch": gb, "avg_launch_us": g["us_cold"]},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    if out["argmax_128256"]["token"] != 2003:
        raise RuntimeError("argmax: planted tie not resolved to the lowest index")
    return 0


BATCH = 64                      # sequences per batched step
CTX_LO, CTX_HI = 512, 8192      # their context lengths, uniform
BATCH_STEPS = 128               # steps the batched workload runs


def kv_position_bytes(s) -> int:
    """Bytes one position's K or V row takes in one layer: n_kv * head_dim elements of the cache dtype, and
    for the int8 cache one code each plus an fp32 scale per K/V head."""
    kvd = s.n_kv * s.head_dim
    return kvd + 4 * s.n_kv if s.kv_dtype == "q8" else kvd * (2 if s.kv_dtype == "bf16" else 4)


def batched_step_bytes(s, ctxs, i) -> int:
    """Algorithmic HBM bytes of batched step i (row r attends ctx_r + i + 1 positions): every weight once,
    each row's embedding row and attended K/V, the appended K/V, the gains."""
    wsz = 2
    d, qd, kvd, F, V, L = s.d, s.n_head * s.head_dim, s.n_kv * s.head_dim, s.hidden, s.vocab, s.n_layer
    weights = L * (d * qd + 2 * d * kvd + qd * d + 3 * d * F) * wsz + V * d * wsz
    emb = len(ctxs) * d * wsz
    gains = (2 * L + 1) * d * 4
    kvp = kv_position_bytes(s)
    kv = sum(L * (int(c) + i + 1) * 2 * kvp for c in ctxs) + len(ctxs) * L * 2 * kvp
    return weights + emb + gains + kv


def batched_attention_bytes(s, ctxs) -> int:
    """Algorithmic bytes of one batched attention launch at positions ctxs: each row's K and V of ctx + 1
    positions, its raw q|k|v and RoPE row read, its appended K/V and its output written (hi and lo)."""
    kvd, qd = s.n_kv * s.head_dim, s.n_head * s.head_dim
    kvp = kv_position_bytes(s)
    per_row_fixed = (qd + 2 * kvd) * 4 + s.head_dim * 4 + 2 * kvp + qd * 2 * 2
    return sum((int(c) + 1) * 2 * kvp + per_row_fixed for c in ctxs)


def run_batched(args) -> int:
    import torch

    import synth
    import autoregressive_decode_step_amd as llmk
    from autoregressive_decode_step_amd import loader

    s = synth.L8B.with_(name="llama-3-8b-shaped bf16, batched", max_seq=CTX_HI + BATCH_STEPS)
    if args.kv == "q8":
        s = s.with_(name="llama-3-8b-shaped bf16, int8 K/V, batched", kv_dtype="q8")
    steps = args.steps if args.steps != 256 else BATCH_STEPS
    if steps > BATCH_STEPS or args.warmup > BATCH_STEPS:
        print(f"the batched workload has room for {BATCH_STEPS} steps per run", file=sys.stderr)
        return 2
    t_start = time.time()
    log(f"generating {s.name} weights and the K/V source")
    W = synth.model(s, seed=0)
    ctxs = synth.ragged_contexts(BATCH, CTX_LO, CTX_HI, seed=3).tolist()
    src = (synth.kv_prefix_q8 if args.kv == "q8" else synth.kv_prefix)(s, CTX_HI + synth.slot_window(BATCH - 1),
                                                                        seed=2)
    first = synth.prompt(BATCH, s.vocab, stream=13).tolist()
    slots = list(range(BATCH))
    log(f"generated in {time.time() - t_start:.1f} s; uploading")
    cfg = loader.config_from(s)
    model = loader.upload_model(cfg, W)
    if args.paged:
        pool = paged_pool(cfg, BATCH, s.max_seq, [c + BATCH_STEPS for c in ctxs], args.paged)
    else:
        pool = loader.new_pool(cfg, BATCH, s.max_seq)
    src_dev = loader.upload_kv_source(src)
    for r in range(BATCH):
        loader.fill_prefix_window(pool, r, src_dev, synth.slot_window(r), ctxs[r])
    del src_dev
    dec = loader.BatchDecoder(cfg, model, pool, BATCH)
    torch.cuda.synchronize()
    log(f"resident in HBM after {time.time() - t_start:.1f} s (pool {sum(t.numel() for t in pool.k) * 4 / 1e9:.1f} GB)")

    def reset():
        for r in range(BATCH):
            pool.slot_len[r] = ctxs[r]

    def run(n, out):
        reset()
        st = dec.steps(slots, first, ctxs, n, out)
        if st != llmk.OK:
            raise RuntimeError(f"decode_steps_batch: {st} {llmk.status_name(st)}")

    if args.warmup > 0:
        run(args.warmup, torch.zeros(args.warmup * BATCH, dtype=torch.int32, device="cuda"))
    toks = torch.zeros(steps * BATCH, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(steps, toks)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / steps
    total_bytes = sum(batched_step_bytes(s, ctxs, i) for i in range(steps))
    gbps = total_bytes / elapsed / 1e9
    log(f"timed {steps} batched steps: {ms_per_step:.3f} ms/step, {BATCH * steps / elapsed:.0f} tokens/s, "
        f"{gbps:.0f} GB/s algorithmic")

    reset()
    avg_ms = {}
    for k, n in enumerate(llmk.BATCH_KERNEL_CLASSES):
        st, ms = llmk.decode_batch_kernel_time(cfg, model, pool, slots, first, ctxs, k, args.kernel_reps,
                                               dec.tokens_out, dec.ws)
        if st != llmk.OK:
            raise RuntimeError(f"decode_batch_kernel_time({n}): {st} {llmk.status_name(st)}")
        avg_ms[n] = ms
        reset()
    log("avg kernel us: " + ", ".join(f"{n} {v * 1e3:.1f}" for n, v in avg_ms.items()))
    at_bytes = batched_attention_bytes(s, ctxs)
    at_gbps = at_bytes / (avg_ms["attention"] * 1e-3) / 1e9
    per_layer = [n for n in llmk.BATCH_KERNEL_CLASSES if n not in ("norm_final", "head")]
    kernel_sum_ms = sum(avg_ms[n] for n in per_layer) * s.n_layer + avg_ms["norm_final"] + avg_ms["head"]
    tokens = toks.cpu().numpy().reshape(steps, BATCH)

    result = {
        "metric": ("decode tokens/s at batch 64 (8B-shaped, ragged contexts, int8 K/V) + achieved HBM GB/s vs peak"
                   if args.kv == "q8" else
                   "decode tokens/s at batch 64 (8B-shaped, ragged contexts) + achieved HBM GB/s vs peak"),
        "value": BATCH * steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama-3-8b-shaped greedy decode, 64 sequences per step, contexts uniform in "
                               "512..8192 (seeded), bf16 weights, " + ("int8 K/V rows with an fp32 scale each"
                                                                        if args.kv == "q8" else "bf16 K/V")
                               + ", projections on bf16 matrix cores",
                   "batch": BATCH, "contexts_mean": float(sum(ctxs) / BATCH), "contexts_min": min(ctxs),
                   "contexts_max": max(ctxs), "weights": "bf16", "kv": args.kv, "accumulation": "f32",
                   "activations_into_mfma": "bf16 hi + lo",
                   "kv_pool": (f"paged, {args.paged}-position blocks, every slot's blocks interleaved with the "
                               f"others'" if args.paged else "contiguous slots")},
        "step_hbm_gbps": gbps,
        "step_frac_of_peak": gbps / PEAK_HBM_GBPS,
        "step_bytes_mean": total_bytes / steps,
        "roofline": {"bound": "hbm", "kernel": "batched attention (attn_kernel, 64 rows)", "achieved": at_gbps,
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": at_gbps / PEAK_HBM_GBPS, "traffic": None,
                     "bytes_per_launch": at_bytes, "avg_launch_us": avg_ms["attention"] * 1e3},
        "kernels_avg_us": {n: v * 1e3 for n, v in avg_ms.items()},
        "kernel_sum_ms_per_step": kernel_sum_ms,
        "first_tokens_row0": tokens[:8, 0].tolist(),
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = [0, 1]
        n = 2
        log(f"oracle baseline: {len(rows)} rows x {n} steps on the host cores")
        m = oracle.Model(s, W)
        tc0 = time.perf_counter()
        agree = True
        for r in rows:
            c = m.new_cache(ctxs[r] + n)
            st0 = synth.slot_window(r)
            def win(x):
                return tuple(a[st0:st0 + ctxs[r]] for a in x) if isinstance(x, tuple) else x[st0:st0 + ctxs[r]]
            c.fill_prefix([(win(k), win(v)) for k, v in src])
            t = first[r]
            for i in range(n):
                lg, _ = m.forward_token(t, ctxs[r] + i, c)
                t = oracle.argmax(lg)[0]
                agree = agree and (t == int(tokens[i, r]))
        tc = time.perf_counter() - tc0
        result["cpu_baseline"] = {"value": len(rows) * n / tc, "unit": "tokens/s", "cores": oracle.lib().orc_num_threads(),
                                  "kind": "oracle",
                                  "sample": f"rows {rows} of the same batch, {n} greedy steps each, one row at a time "
                                            f"(fp64, OpenMP)",
                                  "tokens_agree_with_gpu": agree}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    log(f"total {time.time() - t_start:.1f} s")
    return 0


if __name__ == "__main__":
    sys.exit(main())
