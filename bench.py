#!/usr/bin/env python3
"""Committed tokens/s of the ALoDLM adaptively looped denoising step at 8B shape on one MI355X.

One "step" is one alodlm_denoise_step over the whole batch: Prelude once, then per loop the
shared Core, the Coda, the LM-head / ExitGate readout, the commit rule, compaction and the
Eq. 3 reset, until every sequence halts.  Inputs (random-init weights, prefix ids, planted
readout boosts) are synthetic and already resident in HBM; the prefix cache is built by
alodlm_prefill_kv before timing (reported separately as prefill_ms).

Prints one JSON line.  Options: --gpus (1 only), --steps, --warmup, --workload, --no-cpu-baseline.
"""
import argparse
import json
import os
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores
# HBM bytes per launch of the gate/up GEMM measured with rocprofv3 FETCH_SIZE + WRITE_SIZE (copy-
# calibrated), for the kernel named here; None until the counters are taken on this kernel.
GATE_UP_KERNEL = "k_gemm_pipe<128, 192, 4, 2, 4, 3, false>"
GATE_UP_TRAFFIC_BYTES = 222.8e6


def progress(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def ffn_gate_up_traffic(w, rows_total, launches):
    """Algorithmic HBM bytes per gate/up GEMM launch: the [2F][d] bf16 weight read once, the
    bf16 input rows read once, the bf16 SwiGLU output written once (averaged over launches)."""
    D = w.dims
    wbytes = 2 * D.ffn * D.d_model * 2
    return (launches * wbytes + rows_total * (D.d_model + D.ffn) * 2) / launches


def algorithmic_work(w, loops):
    """Algorithmic HBM bytes and flops per step of each kernel class (what the method must move
    and compute: weights streamed once per layer call, K/V read once per attention call,
    activations read and written once; split-K partials and other implementation traffic are
    not counted).  Rows per loop from the sequences' loop counts; readout rows bounded by the
    looping rows."""
    D = w.dims
    d, hd, F, V = D.d_model, D.head_dim, D.ffn, D.vocab
    Hq, Hkv = D.n_q_heads, D.n_kv_heads
    qkv = (Hq + 2 * Hkv) * hd
    calls = [(w.batch, D.n_pre)] + [(sum(1 for l in loops if l >= s), D.n_core + D.n_coda)
                                     for s in range(1, max(loops) + 1)]
    acc = {k: [0.0, 0.0] for k in ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention", "lm_head",
                                   "norm_rope")}

    def add(k, b, f):
        acc[k][0] += b
        acc[k][1] += f
    for s_idx, (nseq, n_calls) in enumerate(calls):
        R = nseq * w.block
        for _ in range(n_calls):
            add("gemm_qkv", d * qkv * 2 + R * d * 2 + R * qkv * 4, 2.0 * R * d * qkv)
            add("gemm_o", Hq * hd * d * 2 + R * Hq * hd * 2 + R * d * 8, 2.0 * R * Hq * hd * d)
            add("gemm_gate_up", 2 * F * d * 2 + R * d * 2 + R * F * 2, 4.0 * R * d * F)
            add("gemm_down", F * d * 2 + R * F * 2 + R * d * 8, 2.0 * R * F * d)
            add("attention", nseq * Hkv * (w.prefix + w.block) * hd * 4 + R * Hq * hd * 4,
                4.0 * R * Hq * hd * (w.prefix + w.block))
            add("norm_rope", R * (d * 12 + qkv * 6), 0.0)
        if s_idx > 0:
            add("lm_head", d * V * 2 + R * d * 2, 2.0 * R * d * V)
            add("norm_rope", R * d * 6, 0.0)
    return acc


def cpu_baseline(w, tau):
    """The fp64 oracle (as it stands) on a bounded sample: sequence 0 of the same step, over a
    synthetic prefix cache (the prefill is excluded on both sides)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    from oracle import run as orun
    cores = len(os.sched_getaffinity(0))
    ws = replace(w, kv="synthetic", tau_ent=tau, batch=1)
    progress("cpu baseline: generating host weights")
    W = orun.weights(ws)
    cache = orun.cache_for(ws, W, 0)
    progress("cpu baseline: oracle step of one sequence on %d cores" % cores)
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        res = orun.step(ws, W=W, seqs=[0], caches={0: cache})
        el = time.perf_counter() - t0
    committed = int(np.count_nonzero(res[0]["commit_loop"]))
    return dict(value=committed / el, unit="committed tokens/s", cores=cores, kind="oracle",
                sample="sequence 0 of the %s step (1 of %d sequences, %d loops, %d committed), synthetic prefix "
                       "cache, %.1f s" % (w.name, w.batch, res[0]["loops"], committed, el))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="report the step (headline, tau sweep, kernel classes) only: no depth-on-demand prefill, "
                         "sampled commits, outer loop, fp8 K/V or depth eviction sections (for profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain 1 GiB device copy (known traffic, for calibrating HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the step has no cross-GPU path (sequences shard by data "
              "parallelism with no exchange); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from adaptive_looped_denoising_amd import binding as B
    from adaptive_looped_denoising_amd import synth
    from adaptive_looped_denoising_amd.engine import Engine

    w = synth.workload(args.workload)
    taus = synth.TAU_SWEEP_8B if args.workload == "qwen3_8b" else (w.tau_ent,)
    if args.copy_probe:
        src = torch.ones(2 ** 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    progress("workload %s: building engine (device-filled weights)" % w.name)
    # room to append the decoded block at the end; the prefix state kept for depth-on-demand builds
    e = Engine(w, max_prefix=w.prefix + w.block, depth_on_demand=True)
    torch.cuda.synchronize()
    # first-token latency: the depth-on-demand build (depth 1), its deepening to K, then the full
    # prefill that the timed steps use
    prefill_d1_ms = deepen_ms = None
    if not args.step_only:
        e.prefill(depth=1)   # warm-up (first launches of every prefill kernel)
        t0 = time.perf_counter()
        e.prefill(depth=1)
        prefill_d1_ms = (time.perf_counter() - t0) * 1e3
        t0 = time.perf_counter()
        e.deepen(w.k_max)
        deepen_ms = (time.perf_counter() - t0) * 1e3
    progress("prefill")
    t0 = time.perf_counter()
    e.prefill()
    torch.cuda.synchronize()
    prefill_ms = (time.perf_counter() - t0) * 1e3
    progress("prefill %.1f ms (depth 1 first: %s ms, then deepening to %d: %s ms)" % (
        prefill_ms, prefill_d1_ms, w.k_max, deepen_ms))

    def timed(tau, steps, warmup, sample=None, engine=None):
        e_ = e if engine is None else engine
        a = e_.make_args(tau_ent=tau, sample=sample)
        o = e_.make_out(a.k_loops)
        for _ in range(warmup):
            e_.run(a, o)
        torch.cuda.synchronize()
        committed = 0
        loops = []
        t = time.perf_counter()
        for _ in range(steps):
            e_.run(a, o)
            committed += o.n_committed
        torch.cuda.synchronize()
        el = time.perf_counter() - t
        loops = e_.out_loops.cpu().numpy().astype(int).tolist()
        return dict(tok_s=committed / el, ms_per_step=el / steps * 1e3, committed_per_step=committed / steps,
                    loops=loops)

    sweep = {}
    for tau in taus:
        sweep[str(tau)] = timed(tau, args.steps, args.warmup)
        progress("tau_ent %.1f: %s" % (tau, sweep[str(tau)]))
    head = sweep[str(w.tau_ent)]

    # Kernel timing pass: the same steps with HIP event pairs around every kernel class on the
    # library's stream (the stream every kernel of the step runs on).
    B.timing_enable(e.ctx, True)
    prof = timed(w.tau_ent, args.steps, 0)
    kt = B.timing_read(e.ctx)
    B.timing_enable(e.ctx, False)
    loops = prof["loops"]
    D = w.dims
    launches = kt["gemm_gate_up"][1]
    rows_per_step = D.n_pre * w.batch * w.block + (D.n_core + D.n_coda) * w.block * sum(loops)
    per_launch_ms = kt["gemm_gate_up"][0] / max(launches, 1)
    traffic = ffn_gate_up_traffic(w, rows_per_step * args.steps, launches)
    achieved = traffic / (per_launch_ms * 1e-3) / 1e9
    work = algorithmic_work(w, loops)
    # the headline step's decisions (every timed step takes the same ones), for the eviction section
    tok_full, cl_full = e.out_tokens.cpu().numpy(), e.out_cl.cpu().numpy()
    sampled = outer = kv_fp8 = kv_evict = None
    if not args.step_only:
        # Sampled commits (Gumbel-max draws in the LM-head epilogue): the same step and timing pass
        # with ALODLM_STEP_SAMPLE, reported beside the greedy headline.
        samp = timed(w.tau_ent, args.steps, 1, sample=dict(seed=2024, step=0))
        B.timing_enable(e.ctx, True)
        samp_prof = timed(w.tau_ent, args.steps, 0, sample=dict(seed=2024, step=0))
        skt = B.timing_read(e.ctx)
        B.timing_enable(e.ctx, False)
        progress("sampled commits: %s" % samp)
        sampled = dict(tok_s=samp["tok_s"], ms_per_step=samp["ms_per_step"], committed_per_step=samp["committed_per_step"],
                       lm_head_ms_per_step=skt["lm_head"][0] / args.steps,
                       lm_head_ms_per_step_greedy=kt["lm_head"][0] / args.steps,
                       timing_pass_ms_per_step=samp_prof["ms_per_step"])
        # Outer loop: the whole block decoded (steps until no [MASK]), then appended to the cache
        # (the cache grows by one block, so this runs last).
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        blk = e.denoise_block(tau_ent=w.tau_ent)
        blk_s = time.perf_counter() - t0
        masked = int((synth.block_ids(w) == w.mask_id).sum())
        t0 = time.perf_counter()
        e.extend(blk["tokens"])
        ext_s = time.perf_counter() - t0
        outer = dict(masked_tokens=masked, committed=blk["n_committed"], steps=blk["n_steps"], ms=blk_s * 1e3,
                     tok_s=blk["n_committed"] / blk_s, append_ms=ext_s * 1e3,
                     append_rows_per_s=w.batch * w.block / ext_s,
                     append_layer_calls=D.n_pre + w.k_max * D.n_core + D.n_coda)
        progress("outer loop: %s" % outer)
        # fp8 (E4M3) keys and values: the same step on a second engine whose cache and own-block K/V
        # are stored in one byte per element
        e.close()
        del e
        torch.cuda.empty_cache()
        progress("fp8 K/V engine")
        e8 = Engine(replace(w, kv_dtype="fp8"))
        e8.prefill()
        f8 = timed(w.tau_ent, args.steps, args.warmup, engine=e8)
        B.timing_enable(e8.ctx, True)
        timed(w.tau_ent, args.steps, 0, engine=e8)
        kt8 = B.timing_read(e8.ctx)
        B.timing_enable(e8.ctx, False)
        kv_bytes = 2 * D.kv_slots(w.k_max) * w.batch * w.prefix * D.n_kv_heads * D.head_dim
        kv_fp8 = dict(tok_s=f8["tok_s"], ms_per_step=f8["ms_per_step"], committed_per_step=f8["committed_per_step"],
                      attention_ms_per_step=kt8["attention"][0] / args.steps,
                      attention_ms_per_step_bf16=kt["attention"][0] / args.steps,
                      cache_bytes=kv_bytes, cache_bytes_bf16=2 * kv_bytes)
        progress("fp8 K/V: %s" % kv_fp8)
        e8.close()
        del e8
        # Depth eviction: engines whose cache keeps Core depths 1..D only (loops past D read depth D),
        # with the cache bytes they hold and the share of positions both steps commit that get the
        # same token as on the full-depth cache
        kv_evict = {}
        plane = 2 * w.batch * w.prefix * D.n_kv_heads * D.head_dim * 2      # K and V of one slot, bf16
        for keep in (2, 1):
            torch.cuda.empty_cache()
            ev = Engine(replace(w, cache_depths=keep))
            ev.prefill()
            t0 = time.perf_counter()
            ev.prefill()
            torch.cuda.synchronize()
            pf_ms = (time.perf_counter() - t0) * 1e3
            fe = timed(w.tau_ent, args.steps, args.warmup, engine=ev)
            tok, cl = ev.out_tokens.cpu().numpy(), ev.out_cl.cpu().numpy()
            both = (cl != 0) & (cl_full != 0)
            kv_evict["keep_%d" % keep] = dict(
                tok_s=fe["tok_s"], ms_per_step=fe["ms_per_step"], committed_per_step=fe["committed_per_step"],
                loops=fe["loops"], prefill_ms=pf_ms, cache_bytes=plane * (D.kv_slots(keep) + 1),
                cache_bytes_full=plane * D.kv_slots(w.k_max),
                token_agreement=float((tok[both] == tok_full[both]).mean()) if both.any() else None)
            progress("depth eviction, %d kept: %s" % (keep, kv_evict["keep_%d" % keep]))
            ev.close()
            del ev
    kernels = {}
    for k, v in kt.items():
        ms = v[0] / args.steps
        ent = dict(ms_per_step=ms, launches_per_step=v[1] / args.steps)
        if k in work and ms > 0:
            b, f = work[k]
            ent.update(alg_bytes_per_step=b, alg_flops_per_step=f, achieved_gbs=b / (ms * 1e-3) / 1e9,
                       achieved_tflops=f / (ms * 1e-3) / 1e12, hbm_frac=b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                       mfma_frac=f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)
        kernels[k] = ent

    line = {
        "metric": "committed tokens/s per GPU, 8B-shape looped denoise; % MFMA peak + % HBM BW",
        "value": head["tok_s"],
        "unit": "committed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random-init weights and prefix ids, planted readout boosts)",
        "config": {"workload": "%s: Qwen3-8B dims, batch %d, prefix %d, block %d masked, K_max %d, tau_ent %.1f, "
                               "tau_halt %.1f" % (w.name, w.batch, w.prefix, w.block, w.k_max, w.tau_ent, w.tau_halt),
                   "batch": w.batch, "prefix": w.prefix, "block": w.block, "k_max": w.k_max,
                   "tau_ent": w.tau_ent, "tau_halt": w.tau_halt, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": GATE_UP_TRAFFIC_BYTES if w.name == "qwen3_8b" and GATE_UP_TRAFFIC_BYTES else None,
                     "kernel": "FFN gate/up GEMM + SwiGLU (%s), %d rows/launch avg, %.1f us/launch, %.1f MB "
                               "algorithmic per launch" % (GATE_UP_KERNEL, rows_per_step / max(launches / args.steps, 1),
                                                           per_launch_ms * 1e3, traffic / 1e6)},
        "tau_sweep": sweep,
        "sampled_commits": sampled,
        "outer_loop": outer,
        "kv_fp8": kv_fp8,
        "kv_evict": kv_evict,
        "prefill_ms": prefill_ms,
        "prefill_depth_on_demand": None if args.step_only else {
            "depth1_ms": prefill_d1_ms, "deepen_to_kmax_ms": deepen_ms, "prefix_tokens": w.batch * w.prefix},
        # per class: event-timed ms (the event pairs add a little time to short kernels, so the
        # fractions are lower bounds) with algorithmic bytes / flops and their roofline fractions
        "kernels": kernels,
        "timing_pass_ms_per_step": prof["ms_per_step"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, w.tau_ent)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
