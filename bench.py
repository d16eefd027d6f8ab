#!/usr/bin/env python3
"""Throughput of the Llama-3-8B-shaped decoder forward on one MI355X.

Headline (``value``): causal prefill tokens/s of one batch-1, 2048-token sequence through
the 32-layer 8B-shaped stack to the last token's logits (bf16 weights, fp32 accumulation),
with the step's share of the bf16 dense MFMA peak.  ``decode``: greedy KV-cache decode
tokens/s for 32 sequences whose caches hold 4096 prefilled positions, 128 steps, with the
step's share of peak HBM bandwidth.  Inputs are seeded synthetic tensors already resident
in HBM when timing starts.  ``roofline`` is the prefill's dominant kernel (the W1/W3
projection with SiLU*up), timed with HIP events on the launch stream during the timed
steps.  ``cpu_baseline`` times the CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "prefill tokens/s (%MFMA peak) + decode tokens/s (%HBM BW), 8B-shape, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prefill_flops(spec, B: int, S: int) -> float:
    """Algorithmic FLOPs of one prefill: layer GEMMs for every token, the causal lower
    triangle of attention, and the vocabulary projection of the last token."""
    D, H, G, d, F = spec.dim, spec.n_heads, spec.n_kv_heads, spec.head_dim, spec.ffn_hidden
    per_tok = 2 * (D * (H + 2 * G) * d + H * d * D + 3 * D * F)
    attn = 4 * H * d * B * S * (S + 1) / 2        # QK^T and PV, lower triangle incl. diagonal
    return spec.n_layers * (B * S * per_tok + attn) + 2 * B * spec.vocab_size * D


def chunk_prefill_flops(spec, S: int, start_pos: int) -> float:
    """Algorithmic FLOPs of one sequence's S tokens at positions start_pos..: layer GEMMs,
    attention of each token over positions 0..its own, the last token's vocabulary row."""
    D, H, G, d, F = spec.dim, spec.n_heads, spec.n_kv_heads, spec.head_dim, spec.ffn_hidden
    per_tok = 2 * (D * (H + 2 * G) * d + H * d * D + 3 * D * F)
    keys = S * start_pos + S * (S + 1) / 2
    return spec.n_layers * (S * per_tok + 4 * H * d * keys) + 2 * spec.vocab_size * D


def ragged_decode_bytes(spec, positions, steps: int) -> float:
    """decode_bytes for sequences at their own positions (context = position + 1)."""
    D, H, G, d, F, V = (spec.dim, spec.n_heads, spec.n_kv_heads, spec.head_dim,
                        spec.ffn_hidden, spec.vocab_size)
    w_layer = 2 * (D * (H + 2 * G) * d + H * d * D + 3 * D * F + 2 * D)
    weights = spec.n_layers * w_layer + 2 * V * D + 2 * D
    B = len(positions)
    total = 0.0
    for k in range(steps):
        ctx = sum(p + 1 + k for p in positions)
        total += (weights + spec.n_layers * G * ctx * d * 2 * 2
                  + spec.n_layers * B * G * d * 2 * 2 + B * V * 4)
    return total


def decode_bytes(spec, B: int, ctx_first: int, steps: int) -> float:
    """Algorithmic HBM bytes of `steps` decode steps: every weight once per step, the KV
    cache read over the context, the new K/V written, the logits written."""
    D, H, G, d, F, V = (spec.dim, spec.n_heads, spec.n_kv_heads, spec.head_dim,
                        spec.ffn_hidden, spec.vocab_size)
    w_layer = 2 * (D * (H + 2 * G) * d + H * d * D + 3 * D * F + 2 * D)
    weights = spec.n_layers * w_layer + 2 * V * D + 2 * D
    total = 0.0
    for k in range(steps):
        ctx = ctx_first + k
        kv_read = spec.n_layers * B * G * ctx * d * 2 * 2
        kv_write = spec.n_layers * B * G * d * 2 * 2
        total += weights + kv_read + kv_write + B * V * 4
    return total


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILES = {
    "ffn_up": os.path.join(ROOT, "profiles", "ffn_up_gemm_8b_prefill_s2048_traffic.txt"),
    "attention_decode": os.path.join(ROOT, "profiles", "decode_attention_8b_b32_ctx4096_traffic.txt"),
}


def kernel_source_hash() -> str:
    """sha256 over the HIP sources; a traffic figure is only reported for the sources it
    was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "llama_decoder_forward_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".hpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()


def measured_traffic(kind: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary, or
    None if there is none or the kernel sources changed since it was taken."""
    path = TRAFFIC_FILES[kind]
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(spec, seed: int, S: int, n_layers_sample: int, dec_ctx: int, n_dec_layers: int = 4):
    """Time the CPU oracle (float32) on bounded samples of the workloads:

    * prefill of 1 x S tokens through `n_layers_sample` of the layers plus the head, the
      per-layer time scaled to the whole stack (``value``, tokens/s);
    * one decode step of one sequence at position `dec_ctx` over a cache of `dec_ctx`
      positions (random keys and values: the time does not depend on them) through
      `n_dec_layers` layers plus the head, scaled to the whole stack (``decode``; the oracle
      decodes the rows of a batch one after the other, so this is its tokens/s at any batch);
    * one layer at 17 tokens (``layer_17``).
    ``cores`` is the number of BLAS threads the oracle's matrix products used,
    ``affinity_cores`` the host cores this process may run on."""
    import dataclasses
    from oracle import llama_oracle as O
    from llama_decoder_forward_amd import synthetic as syn
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = affinity
    synth = syn.SyntheticWeights(spec, seed, cache=False)
    names = ["tok_embeddings.weight", "norm.weight", "output.weight"]
    for l in range(n_layers_sample):
        names += [n for n, *_ in syn.layer_weight_specs(spec, l)]
    W = {n: synth.as_float(n, np.float32) for n in names}
    toks = syn.tokens(seed, 1, S, spec.vocab_size)[0]
    t0 = time.perf_counter()
    x = O.embed(toks, W, np.float32)
    cache = O.SequenceCache(spec, S, np.float32)
    t1 = time.perf_counter()
    for l in range(n_layers_sample):
        x = O.layer_forward(x, W, spec, l, cache, 0)
    t2 = time.perf_counter()
    logits = O.head_logits(x[-1:], W, spec)
    t3 = time.perf_counter()
    assert np.isfinite(logits).all()
    per_layer = (t2 - t1) / n_layers_sample
    est = (t1 - t0) + per_layer * spec.n_layers + (t3 - t2)
    del cache

    # decode: one token at position ctx over ctx cached positions, through the layers
    # already loaded, scaled to the whole stack
    n_dec_layers = min(n_dec_layers, n_layers_sample)
    dspec = dataclasses.replace(spec, n_layers=n_dec_layers)

    def decode_step_time(ctx):
        dcache = O.SequenceCache(dspec, ctx + 1, np.float32)
        for l in range(n_dec_layers):
            dcache.k[l][:, :ctx] = syn.normal(seed, f"cpu.k{l}", (spec.n_kv_heads, ctx, spec.head_dim))
            dcache.v[l][:, :ctx] = syn.normal(seed, f"cpu.v{l}", (spec.n_kv_heads, ctx, spec.head_dim))
        d0 = time.perf_counter()
        xd = O.embed(toks[:1], W, np.float32)
        d1 = time.perf_counter()
        for l in range(n_dec_layers):
            xd = O.layer_forward(xd, W, dspec, l, dcache, ctx)
        d2 = time.perf_counter()
        lg = O.head_logits(xd, W, spec)
        d3 = time.perf_counter()
        assert np.isfinite(lg).all()
        return (d1 - d0) + (d2 - d1) / n_dec_layers * spec.n_layers + (d3 - d2), d3 - d0

    dec_step, d_meas = decode_step_time(dec_ctx)
    long_ctx = 8192
    dec_long, dl_meas = decode_step_time(long_ctx)

    # one layer at 17 tokens
    x17 = syn.normal(2, "x", (17, spec.dim))
    c17 = O.SequenceCache(dataclasses.replace(spec, n_layers=1), 17, np.float32)
    l0 = time.perf_counter()
    O.layer_forward(x17, W, spec, 0, c17, 0)
    l1 = time.perf_counter()
    return {"value": S / est, "unit": "tokens/s", "cores": int(cores),
            "affinity_cores": int(affinity), "kind": "oracle",
            "sample": (f"prefill of 1 x {S} tokens through {n_layers_sample} of "
                       f"{spec.n_layers} layers plus the head in float32 "
                       f"({t3 - t0:.1f} s measured); per-layer time scaled to "
                       f"{spec.n_layers} layers"),
            "seconds_measured": t3 - t0 + d_meas + dl_meas + l1 - l0,
            "decode": {"value": 1.0 / dec_step, "unit": "tokens/s",
                       "ms_per_token": dec_step * 1e3,
                       "sample": (f"one decode step of one sequence at position {dec_ctx} through "
                                  f"{n_dec_layers} of {spec.n_layers} layers plus the head in "
                                  f"float32 ({d_meas:.2f} s measured); per-layer time scaled; "
                                  f"the oracle decodes the rows of a batch one after the other")},
            "decode_long_context": {"value": 1.0 / dec_long, "unit": "tokens/s",
                                    "ms_per_token": dec_long * 1e3,
                                    "sample": (f"the same at position {long_ctx} "
                                               f"({dl_meas:.2f} s measured)")},
            "layer_17": {"ms": (l1 - l0) * 1e3,
                         "sample": "one 8B-shaped layer at 1 x 17 tokens in float32"}}


def long_context(spec, weights, prefill_runs: int, decode_steps: int) -> dict:
    """4 sequences of 8192 tokens prefilled in one call (timed over prefill_runs calls after
    one warmup), then decode_steps greedy steps of the batch against those caches
    (llama_generate, timed after one warmup); a model of its own, with the cache sized for
    8192 + decode_steps positions."""
    import torch
    from llama_decoder_forward_amd import binding as bd
    from llama_decoder_forward_amd import synthetic as syn

    L_B, L_S = 4, 8192
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ml = bd.Model(spec, weights, max_batch=L_B, max_seq=L_S + decode_steps, max_tokens=L_B * L_S)
    ltoks = torch.from_numpy(syn.tokens(5, L_B, L_S, spec.vocab_size)).cuda()
    ml.prefill(ltoks)                                 # warmup
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(prefill_runs):
        ml.prefill(ltoks)
    stop.record(stream)
    torch.cuda.synchronize()
    lp_ms = start.elapsed_time(stop) / prefill_runs
    _, first = ml.prefill(ltoks, want_next=True)      # untimed: the first greedy tokens
    ml.generate(first, L_S, decode_steps)             # warmup (same positions)
    torch.cuda.synchronize()
    start.record(stream)
    ml.generate(first, L_S, decode_steps)
    stop.record(stream)
    torch.cuda.synchronize()
    ld_ms = start.elapsed_time(stop)
    ml.sync_status()
    ml.free()
    lfl = prefill_flops(spec, L_B, L_S)
    lbytes = decode_bytes(spec, L_B, L_S + 1, decode_steps)
    log(f"long context: prefill {lp_ms:.1f} ms, decode {ld_ms / decode_steps:.3f} ms/step")
    return {
        "workload": f"llama3-8b-shaped prefill of {L_B} x {L_S} tokens in one call, then "
                    f"{decode_steps} greedy decode steps of the batch (llama_generate)",
        "prefill": {"value": L_B * L_S / (lp_ms * 1e-3), "unit": "tokens/s",
                    "ms_per_step": lp_ms, "steps": prefill_runs,
                    "mfma_frac": lfl / (lp_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                    "tflops": lfl / (lp_ms * 1e-3) / 1e12},
        "decode": {"value": L_B * decode_steps / (ld_ms * 1e-3), "unit": "tokens/s",
                   "ms_per_step": ld_ms / decode_steps, "steps": decode_steps, "batch": L_B,
                   "context": [L_S + 1, L_S + decode_steps],
                   "hbm_gbs": lbytes / (ld_ms * 1e-3) / 1e9,
                   "hbm_frac": lbytes / (ld_ms * 1e-3) / 1e9 / PEAK_HBM_GBS},
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5, help="timed prefill steps")
    ap.add_argument("--warmup", type=int, default=2, help="untimed prefill steps")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--decode-batch", type=int, default=32)
    ap.add_argument("--decode-ctx", type=int, default=4096)
    ap.add_argument("--seq", type=int, default=2048)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context leg (4 x 8192 prefill, then batch-4 decode)")
    ap.add_argument("--long-only", action="store_true",
                    help="run only the long-context leg, short (1 timed prefill, 8 decode steps), "
                         "and print its object; for rocprofv3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-layers", type=int, default=10)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--print-source-hash", action="store_true")
    ap.add_argument("--profile-only", action="store_true",
                    help="a short run for rocprofv3: 1 warmup + --steps prefill, 8 decode steps, "
                         "no long-context leg and no CPU baseline")
    args = ap.parse_args()

    if args.print_source_hash:
        print(kernel_source_hash())
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr, flush=True)
        return 2

    import torch
    from llama_decoder_forward_amd import binding as bd
    from llama_decoder_forward_amd import synthetic as syn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB (1073741824 bytes) device to device for counter calibration")
        del src, dst
    spec = syn.LLAMA3_8B
    seed = 3
    if args.long_only:
        weights = bd.upload_weights(syn.SyntheticWeights(spec, seed, cache=False))
        print(json.dumps({"long_context": long_context(spec, weights, prefill_runs=1,
                                                       decode_steps=8)}), flush=True)
        return 0
    dec_B, dec_ctx, dec_steps = args.decode_batch, args.decode_ctx, args.decode_steps
    if args.profile_only:
        dec_steps = min(dec_steps, 8)
    run_decode = not args.no_decode
    max_batch = dec_B if run_decode else 1
    max_seq = max(args.seq, dec_ctx + dec_steps if run_decode else 0)
    max_tokens = max(args.seq, dec_B * dec_ctx if run_decode else 0)

    t = time.perf_counter()
    synth = syn.SyntheticWeights(spec, seed, cache=False)
    weights = bd.upload_weights(synth)
    torch.cuda.synchronize()
    log(f"weights generated and uploaded in {time.perf_counter() - t:.1f} s")
    m = bd.Model(spec, weights, max_batch=max_batch, max_seq=max_seq, max_tokens=max_tokens)

    # ---------------------------------------------------------------- prefill (headline)
    S = args.seq
    toks = torch.from_numpy(syn.tokens(seed, 1, S, spec.vocab_size)).cuda()
    stream = torch.cuda.current_stream()
    warm = 1 if args.profile_only else args.warmup
    for _ in range(warm):
        m.prefill(toks)
    torch.cuda.synchronize()
    log("prefill warmup done")
    m.profile_kernel("ffn_up")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        m.prefill(toks)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps
    k_ms, k_n = m.profile_read()
    m.profile_kernel("none")
    m.sync_status()
    log(f"prefill: {ms_step:.2f} ms/step")
    flops = prefill_flops(spec, 1, S)
    ffn_up_flops = 2 * S * 2 * spec.ffn_hidden * spec.dim
    k_avg = k_ms / max(k_n, 1)
    ach = ffn_up_flops / (k_avg * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": S / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3-8b-shaped causal prefill: 32 layers + lm_head of the last "
                               "token, batch 1 x 2048 tokens",
                   "batch": 1, "seq_len": S, "parallelism": "none (1 GPU)"},
        "prefill_mfma_frac": flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "prefill_tflops": flops / (ms_step * 1e-3) / 1e12,
        "roofline": {"kernel": "ffn_up (W1/W3 GEMM + SiLU*up), M=2048 N=2x14336 K=4096",
                     "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("ffn_up"),
                     "avg_launch_ms": k_avg, "launches": k_n},
    }

    # ---------------------------------------------------------------- one layer, 17 tokens
    x17 = torch.from_numpy(syn.normal(2, "x", (1, 17, spec.dim))).cuda()
    y17 = torch.empty_like(x17)
    for _ in range(3):
        m.layer_forward(0, x17, x_out=y17)
    n17 = 5 if args.profile_only else 50
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n17):
        m.layer_forward(0, x17, x_out=y17)
    stop.record(stream)
    torch.cuda.synchronize()
    l17 = start.elapsed_time(stop) / n17
    w_layer_bytes = 2 * (spec.dim * (spec.n_heads + 2 * spec.n_kv_heads) * spec.head_dim
                         + spec.n_heads * spec.head_dim * spec.dim + 3 * spec.dim * spec.ffn_hidden
                         + 2 * spec.dim)
    result["layer_17"] = {
        "workload": "one llama3-8b-shaped decoder layer on 1 x 17 tokens at positions 0..16 "
                    "(llama_layer_forward)",
        "us_per_call": l17 * 1e3, "calls": n17,
        "hbm_gbs": w_layer_bytes / (l17 * 1e-3) / 1e9,
        "hbm_frac": w_layer_bytes / (l17 * 1e-3) / 1e9 / PEAK_HBM_GBS,
    }
    log(f"one layer at 17 tokens: {l17 * 1e3:.1f} us")

    # ---------------------------------------------------------------- decode
    if run_decode:
        dtoks = torch.from_numpy(syn.tokens(4, dec_B, dec_ctx, spec.vocab_size)).cuda()
        t = time.perf_counter()
        _, first = m.prefill(dtoks, want_next=True)
        torch.cuda.synchronize()
        log(f"decode setup prefill ({dec_B} x {dec_ctx}) in {time.perf_counter() - t:.1f} s")
        m.generate(first, dec_ctx, dec_steps)            # warmup (same positions)
        torch.cuda.synchronize()
        start.record(stream)
        out, _ = m.generate(first, dec_ctx, dec_steps)
        stop.record(stream)
        torch.cuda.synchronize()
        dms = start.elapsed_time(stop)
        m.sync_status()
        dbytes = decode_bytes(spec, dec_B, dec_ctx + 1, dec_steps)
        # decode attention kernel timed on separate decode steps
        m.profile_kernel("attention")
        cur = first
        n_eager = 4
        for k in range(n_eager):
            cur, _ = m.decode_step(cur, dec_ctx + k, want_logits=False)
        torch.cuda.synchronize()
        a_ms, a_n = m.profile_read()
        m.profile_kernel("none")
        a_avg = a_ms / max(a_n, 1)
        ctx_mid = dec_ctx + 1 + (n_eager - 1) / 2
        a_bytes = dec_B * spec.n_kv_heads * ctx_mid * spec.head_dim * 2 * 2
        a_gbs = a_bytes / (a_avg * 1e-3) / 1e9
        log(f"decode: {dms / dec_steps:.3f} ms/step")
        result["decode"] = {
            "value": dec_B * dec_steps / (dms * 1e-3), "unit": "tokens/s",
            "ms_per_step": dms / dec_steps, "steps": dec_steps, "batch": dec_B,
            "context": [dec_ctx + 1, dec_ctx + dec_steps],
            "workload": f"llama3-8b-shaped greedy KV-cache decode, batch {dec_B}, "
                        f"{dec_ctx} prefilled positions, {dec_steps} steps (llama_generate)",
            "hbm_gbs": dbytes / (dms * 1e-3) / 1e9,
            "hbm_frac": dbytes / (dms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "roofline": {"kernel": "decode attention (one workgroup per sequence and KV head over its whole context)", "bound": "hbm",
                         "achieved": a_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": a_gbs / PEAK_HBM_GBS,
                         "traffic": measured_traffic("attention_decode"),
                         "avg_launch_ms": a_avg, "launches": a_n},
            "tokens_head": out[:4, 0].tolist(),
        }

        # ragged decode: every sequence at its own position (llama_decode_step_ragged), the
        # contexts spread evenly over [dec_ctx/2, dec_ctx)
        rpos = [dec_ctx - 1 - (b * dec_ctx) // (2 * dec_B) for b in range(dec_B)]
        r_steps = 8 if args.profile_only else 32
        pos_dev = torch.tensor(rpos, dtype=torch.int32, device="cuda")
        cur = first.clone()
        for _ in range(2):    # warmup of the timed loop body, including the position update
            cur, _ = m.decode_step_ragged(cur, pos_dev, want_logits=False)
            pos_dev += 1
        pos_dev -= 2
        cur = first.clone()
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(r_steps):
            cur, _ = m.decode_step_ragged(cur, pos_dev, want_logits=False)
            pos_dev += 1
        stop.record(stream)
        torch.cuda.synchronize()
        rms = start.elapsed_time(stop)
        m.sync_status()
        rbytes = ragged_decode_bytes(spec, rpos, r_steps)
        log(f"ragged decode: {rms / r_steps:.3f} ms/step")
        result["ragged_decode"] = {
            "value": dec_B * r_steps / (rms * 1e-3), "unit": "tokens/s",
            "ms_per_step": rms / r_steps, "steps": r_steps, "batch": dec_B,
            "context": [min(rpos) + 1, max(rpos) + r_steps],
            "workload": f"llama3-8b-shaped greedy decode of {dec_B} sequences at their own "
                        f"positions ({min(rpos)}..{max(rpos)} at the first step), "
                        f"{r_steps} steps (llama_decode_step_ragged, eager)",
            "hbm_gbs": rbytes / (rms * 1e-3) / 1e9,
            "hbm_frac": rbytes / (rms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        }

        # chunked prefill: the second S tokens of a sequence, at positions S..2S-1, after a
        # prefix of S (llama_prefill_at); each call rewrites the same cache entries
        if 2 * S <= max_seq:
            c_toks = torch.from_numpy(syn.tokens(seed + 1, 1, 2 * S, spec.vocab_size)).cuda()
            m.prefill(c_toks[:, :S].contiguous())
            chunk = c_toks[:, S:].contiguous()
            c_steps = 1 if args.profile_only else max(1, args.steps)
            m.prefill(chunk, start_pos=S)
            torch.cuda.synchronize()
            start.record(stream)
            for _ in range(c_steps):
                m.prefill(chunk, start_pos=S)
            stop.record(stream)
            torch.cuda.synchronize()
            cms = start.elapsed_time(stop) / c_steps
            m.sync_status()
            cfl = chunk_prefill_flops(spec, S, S)
            log(f"chunked prefill: {cms:.2f} ms per {S}-token chunk at start_pos {S}")
            result["chunked_prefill"] = {
                "value": S / (cms * 1e-3), "unit": "tokens/s", "ms_per_step": cms,
                "steps": c_steps,
                "workload": f"llama3-8b-shaped prefill of tokens {S}..{2 * S - 1} of one "
                            f"sequence after a {S}-token prefix (llama_prefill_at)",
                "mfma_frac": cfl / (cms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                "tflops": cfl / (cms * 1e-3) / 1e12,
            }

    # ---------------------------------------------------------------- long context
    if not args.no_long and not args.profile_only:
        del m
        torch.cuda.empty_cache()
        result["long_context"] = long_context(spec, weights, prefill_runs=2, decode_steps=64)
        m = None

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline and not args.profile_only:
        log("timing the CPU oracle sample")
        m = None
        del weights
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_baseline(spec, seed, S, args.cpu_layers, dec_ctx)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
