#!/usr/bin/env python3
"""Committed tokens/s of the ALoDLM adaptively looped denoising step at 8B shape on one MI355X.

One "step" is one alodlm_denoise_step over the whole batch: Prelude once, then per loop the
shared Core, the Coda, the LM-head / ExitGate readout, the commit rule, compaction and the
Eq. 3 reset, until every sequence halts.  Inputs (random-init weights, prefix ids, planted
readout boosts) are synthetic and already resident in HBM; the prefix cache is built by
alodlm_prefill_kv before timing (reported separately as prefill_ms).

The headline is the 8B-shape workload (batch 8, prefix 1024, block 32).  The same line carries
the other workloads, each timed the same way with its own kernel-class roofline fractions: the
8B workload with planted boosts strong enough to commit by entropy (a labelled variant), the
1.7B-shape step, the 8B long-context step and the readout microbench (32 / 256 / 2048 rows).

Prints one JSON line.  Options: --gpus (1 only), --steps, --warmup, --workload, --configs,
--no-cpu-baseline, --step-only, --copy-probe.
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
RIDGE = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # flop per byte where the two bounds meet
# HBM bytes per launch of the gate/up GEMM measured with rocprofv3 FETCH_SIZE + WRITE_SIZE
# (copy-calibrated), valid only for this kernel at this mean row count per launch
GATE_UP_COUNTERS = dict(kernel="k_gemm_pipe<128, 192, 4, 2, 4, 3, false>", rows_per_launch=242.6, bytes=223.3e6,
                        profile="profiles/gemm_gate_up_swiglu_qwen3_8b_hbm_traffic.md")
CLASSES = ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down", "attention", "lm_head", "norm_rope")


def progress(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


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
    acc = {k: [0.0, 0.0] for k in CLASSES}

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


def roofline(bytes_, flops, seconds, kernel):
    """Roofline entry of one kernel: bound by its arithmetic intensity against the ridge point."""
    mfma = flops / max(bytes_, 1.0) > RIDGE
    if mfma:
        a = flops / seconds / 1e12
        return dict(bound="mfma", achieved=a, peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=a / BF16_PEAK_TFLOPS,
                    kernel=kernel)
    a = bytes_ / seconds / 1e9
    return dict(bound="hbm", achieved=a, peak=HBM_PEAK_GBS, unit="GB/s", frac=a / HBM_PEAK_GBS, kernel=kernel)


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
        res = orun.step(ws, W=W, seqs=[0], caches={0: cache}, exit_b=w.exit_bias())
        el = time.perf_counter() - t0
    committed = int(np.count_nonzero(res[0]["commit_loop"]))
    return dict(value=committed / el, unit="committed tokens/s", cores=cores, kind="oracle",
                sample="sequence 0 of the %s step (1 of %d sequences, %d loops, %d committed), synthetic prefix "
                       "cache, %.1f s" % (w.name, w.batch, res[0]["loops"], committed, el))


class Runner:
    """Times denoising steps of one engine and derives the per-config figures."""

    def __init__(self, e, steps, warmup):
        self.e, self.steps, self.warmup = e, steps, warmup

    def timed(self, tau, sample=None, steps=None, warmup=None):
        import torch
        e = self.e
        steps = self.steps if steps is None else steps
        warmup = self.warmup if warmup is None else warmup
        a = e.make_args(tau_ent=tau, sample=sample)
        o = e.make_out(a.k_loops)
        for _ in range(warmup):
            e.run(a, o)
        torch.cuda.synchronize()
        committed = 0
        t = time.perf_counter()
        for _ in range(steps):
            e.run(a, o)
            committed += o.n_committed
        torch.cuda.synchronize()
        el = time.perf_counter() - t
        loops = e.out_loops.cpu().numpy().astype(int).tolist()
        return dict(tok_s=committed / el, ms_per_step=el / steps * 1e3, committed_per_step=committed / steps,
                    loops=loops)

    def decisions(self, tau):
        """One untimed step with per-loop records: mean first-loop ExitGate lambda over the block rows,
        loops per committed token (each token's commit loop), entropy and forced commits."""
        import numpy as np
        r = self.e.step(tau_ent=tau, records=True)
        lam0 = r.lam[0]
        cl = np.abs(r.commit_loop[r.commit_loop != 0])
        return dict(mean_first_loop_lambda=float(np.nanmean(lam0)), loops_per_token=float(cl.mean()) if cl.size else None,
                    entropy_commits=int((r.commit_loop > 0).sum()), forced_commits=int((r.commit_loop < 0).sum()))

    def kernel_classes(self, tau, steps=None):
        """Per-class event timing over a pass identical to the timed one (HIP events on the library's
        stream around each kernel class), with algorithmic bytes / flops and roofline fractions."""
        from adaptive_looped_denoising_amd import binding as B
        e, w = self.e, self.e.w
        steps = self.steps if steps is None else steps
        B.timing_enable(e.ctx, True)
        prof = self.timed(tau, steps=steps, warmup=0)
        kt = B.timing_read(e.ctx)
        B.timing_enable(e.ctx, False)
        work = algorithmic_work(w, prof["loops"])
        kernels = {}
        for k, (ms_tot, n) in kt.items():
            ms = ms_tot / steps
            ent = dict(ms_per_step=ms, launches_per_step=n / steps)
            if k in work and ms > 0:
                b, f = work[k]
                ent.update(alg_bytes_per_step=b, alg_flops_per_step=f, achieved_gbs=b / (ms * 1e-3) / 1e9,
                           achieved_tflops=f / (ms * 1e-3) / 1e12, hbm_frac=b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           mfma_frac=f / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS)
            kernels[k] = ent
        return prof, kt, kernels

    def gate_up_roofline(self, kt, loops, steps):
        """Roofline of the dominant kernel, the FFN gate/up GEMM + SwiGLU: algorithmic bytes (or flops)
        per launch over its mean event-timed launch duration; the kernel named as the dispatcher
        picks it for each loop's row count."""
        from adaptive_looped_denoising_amd import binding as B
        w = self.e.w
        D = w.dims
        rows = [w.batch * w.block] * D.n_pre + [sum(1 for l in loops if l >= s) * w.block
                                               for s in range(1, max(loops) + 1) for _ in range(D.n_core + D.n_coda)]
        launches = kt["gemm_gate_up"][1] / steps
        per_launch_s = kt["gemm_gate_up"][0] / max(kt["gemm_gate_up"][1], 1) * 1e-3
        mean_rows = sum(rows) / len(rows)
        wbytes = 2 * D.ffn * D.d_model * 2
        bytes_ = wbytes + mean_rows * (D.d_model + D.ffn) * 2
        flops = 4.0 * mean_rows * D.d_model * D.ffn
        scratch = w.batch * w.block * max(2 * D.ffn, D.qkv_out) * 8
        names = sorted({B.gemm_choice(3, r, 2 * D.ffn, D.d_model, scratch)[2] for r in set(rows)})
        rf = roofline(bytes_, flops, per_launch_s, " / ".join(names))
        rf.update(rows_per_launch=mean_rows, launches_per_step=launches, us_per_launch=per_launch_s * 1e6,
                  alg_bytes_per_launch=bytes_, alg_flops_per_launch=flops)
        c = GATE_UP_COUNTERS
        if names == [c["kernel"]] and abs(mean_rows - c["rows_per_launch"]) <= 0.02 * c["rows_per_launch"]:
            rf["traffic"] = c["bytes"]
            rf["traffic_source"] = c["profile"]
        else:
            rf["traffic"] = None
            rf["traffic_note"] = "counters (%s) were taken on %s at %.0f rows per launch" % (
                c["profile"], c["kernel"], c["rows_per_launch"])
        return rf


def step_config(Engine, w, args, taus=None, engine_kw=None, boosts=None):
    """Build, prefill, time and profile one step workload; returns (figures, engine)."""
    import torch
    t0 = time.perf_counter()
    e = Engine(w, **(engine_kw or {}))
    torch.cuda.synchronize()
    progress("%s: engine ready in %.1f s" % (w.name, time.perf_counter() - t0))
    t0 = time.perf_counter()
    e.prefill()
    prefill_ms = (time.perf_counter() - t0) * 1e3
    r = Runner(e, args.steps, args.warmup)
    taus = taus or (w.tau_ent,)
    sweep = {str(t): r.timed(t) for t in taus}
    head = sweep[str(w.tau_ent)]
    prof, kt, kernels = r.kernel_classes(w.tau_ent)
    out = dict(head, prefill_ms=prefill_ms, **r.decisions(w.tau_ent), kernels=kernels,
               roofline=r.gate_up_roofline(kt, prof["loops"], args.steps), timing_pass_ms_per_step=prof["ms_per_step"])
    if len(taus) > 1:
        out["tau_sweep"] = sweep
    progress("%s: %.1f tok/s, %.2f ms/step, loops %s" % (w.name, out["tok_s"], out["ms_per_step"], out["loops"]))
    return out, e, r


def readout_config(Engine, n_rows, args):
    """Readout microbench: LM head over n_rows given rows (4096 x 151936), ExitGate, halting update,
    commit, compaction and the Eq. 3 embedding gather, one call = one readout; the LM head dominates."""
    import numpy as np
    import torch
    from adaptive_looped_denoising_amd import synth
    w = synth.readout_workload(n_rows)
    e = Engine(w)
    rows = synth.readout_rows(n_rows)
    bt, bv = synth.boosts(w)
    rows_d = torch.from_numpy(np.ascontiguousarray(rows).view(np.int16)).cuda().view(torch.bfloat16)
    bt_d, bv_d = torch.from_numpy(bt.reshape(-1)).cuda(), torch.from_numpy(bv.reshape(-1)).cuda()
    group = synth.READOUT_GROUP if n_rows >= synth.READOUT_GROUP else n_rows
    out = e.readout_commit(rows_d, group, w.tau_ent, w.tau_halt, bt_d, bv_d)
    call = lambda: e.readout_commit(rows_d, group, w.tau_ent, w.tau_halt, bt_d, bv_d, out=out)  # noqa: E731
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(st)
    for _ in range(args.steps):
        call()
    ev1.record(st)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) / args.steps * 1e3
    D = w.dims
    bytes_ = D.d_model * D.vocab * 2 + n_rows * D.d_model * 2
    flops = 2.0 * n_rows * D.d_model * D.vocab
    from adaptive_looped_denoising_amd import binding as B
    kernel = B.gemm_choice(2, n_rows, D.vocab, D.d_model, 0)[2]
    lam = out["lam"].cpu().numpy()
    cl = out["commit_loop"].cpu().numpy()
    res = dict(us_per_readout=us, rows_per_s=n_rows / (us * 1e-6), mean_lambda=float(lam.mean()),
               entropy_commits=int((cl > 0).sum()), forced_commits=int((cl < 0).sum()),
               roofline=roofline(bytes_, flops, us * 1e-6, kernel + " + combine, ExitGate, commit, gather"))
    e.close()
    progress("readout %d rows: %.1f us, %s" % (n_rows, us, res["roofline"]))
    return res


def kill_children():
    """Ends any child process this run started (none should outlive the line)."""
    try:
        import psutil
        kids = psutil.Process().children(recursive=True)
        for k in kids:
            k.terminate()
        psutil.wait_procs(kids, timeout=5)
    except Exception:
        pass


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="qwen3_8b")
    ap.add_argument("--configs", default="entropy_commits,qwen3_1p7b,qwen3_8b_long,readout",
                    help="secondary workloads reported beside the headline (comma list; empty for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--step-only", action="store_true",
                    help="report the headline step only: no secondary workloads, depth-on-demand prefill, sampled "
                         "commits, outer loop, fp8 K/V or depth eviction sections (for profiling runs)")
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
    head, e, run = step_config(Engine, w, args, taus=taus,
                               engine_kw=dict(max_prefix=w.prefix + w.block, depth_on_demand=True))
    D = w.dims
    extra = {}
    if not args.step_only:
        # first-token latency: the depth-on-demand build (depth 1), its deepening to K, the full prefill
        e.prefill(depth=1)   # warm-up (first launches of every prefill kernel)
        t0 = time.perf_counter()
        e.prefill(depth=1)
        d1 = (time.perf_counter() - t0) * 1e3
        t0 = time.perf_counter()
        e.deepen(w.k_max)
        dp = (time.perf_counter() - t0) * 1e3
        extra["prefill_depth_on_demand"] = dict(depth1_ms=d1, deepen_to_kmax_ms=dp, prefix_tokens=w.batch * w.prefix)
        e.prefill()
        tok_full, cl_full = e.out_tokens.cpu().numpy(), e.out_cl.cpu().numpy()
        # sampled commits (Gumbel-max draws in the LM-head epilogue), greedy headline beside it
        samp = run.timed(w.tau_ent, sample=dict(seed=2024, step=0))
        B.timing_enable(e.ctx, True)
        run.timed(w.tau_ent, sample=dict(seed=2024, step=0), warmup=0)
        skt = B.timing_read(e.ctx)
        B.timing_enable(e.ctx, False)
        extra["sampled_commits"] = dict(tok_s=samp["tok_s"], ms_per_step=samp["ms_per_step"],
                                        committed_per_step=samp["committed_per_step"],
                                        lm_head_ms_per_step=skt["lm_head"][0] / args.steps,
                                        lm_head_ms_per_step_greedy=head["kernels"]["lm_head"]["ms_per_step"])
        # labelled variant: planted boosts strong enough to commit by entropy at V = 151936, so the
        # commit / compaction path runs at the real shape (tau swept like the headline)
        if "entropy_commits" in args.configs:
            wp = replace(w, boost_lo=10.0, boost_hi=20.0)
            bt, bv = synth.boosts(wp)
            e.boost_tok = torch.from_numpy(bt).to(e.device)
            e.boost_val = torch.from_numpy(bv).to(e.device)
            sweep = {str(t): run.timed(t) for t in taus}
            prof, kt, kernels = run.kernel_classes(w.tau_ent)
            extra["qwen3_8b_entropy_commits"] = dict(
                label="variant: planted boosts beta ~ U(10, 20) instead of U(4, 10)", **sweep[str(w.tau_ent)],
                tau_sweep=sweep, **run.decisions(w.tau_ent), kernels=kernels,
                roofline=run.gate_up_roofline(kt, prof["loops"], args.steps))
            for t in taus:
                extra["qwen3_8b_entropy_commits"]["tau_sweep"][str(t)].update(run.decisions(t))
            progress("entropy-commit variant: %s" % sweep)
            bt, bv = synth.boosts(w)
            e.boost_tok = torch.from_numpy(bt).to(e.device)
            e.boost_val = torch.from_numpy(bv).to(e.device)
        # outer loop: the whole block decoded, then appended to the cache (grows the cache: last)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        blk = e.denoise_block(tau_ent=w.tau_ent)
        blk_s = time.perf_counter() - t0
        t0 = time.perf_counter()
        e.extend(blk["tokens"])
        ext_s = time.perf_counter() - t0
        extra["outer_loop"] = dict(masked_tokens=int((synth.block_ids(w) == w.mask_id).sum()),
                                   committed=blk["n_committed"], steps=blk["n_steps"], ms=blk_s * 1e3,
                                   tok_s=blk["n_committed"] / blk_s, append_ms=ext_s * 1e3,
                                   append_layer_calls=D.n_pre + w.k_max * D.n_core + D.n_coda)
        progress("outer loop: %s" % extra["outer_loop"])
        e.close()
        del e, run
        torch.cuda.empty_cache()
        # fp8 (E4M3) keys and values
        e8 = Engine(replace(w, kv_dtype="fp8"))
        e8.prefill()
        r8 = Runner(e8, args.steps, args.warmup)
        f8 = r8.timed(w.tau_ent)
        _, kt8, _ = r8.kernel_classes(w.tau_ent)
        kv_bytes = 2 * D.kv_slots(w.k_max) * w.batch * w.prefix * D.n_kv_heads * D.head_dim
        extra["kv_fp8"] = dict(tok_s=f8["tok_s"], ms_per_step=f8["ms_per_step"],
                               committed_per_step=f8["committed_per_step"],
                               attention_ms_per_step=kt8["attention"][0] / args.steps,
                               attention_ms_per_step_bf16=head["kernels"]["attention"]["ms_per_step"],
                               cache_bytes=kv_bytes, cache_bytes_bf16=2 * kv_bytes)
        e8.close()
        del e8, r8
        # depth eviction: caches keeping Core depths 1..D only
        extra["kv_evict"] = {}
        plane = 2 * w.batch * w.prefix * D.n_kv_heads * D.head_dim * 2
        for keep in (2, 1):
            torch.cuda.empty_cache()
            ev = Engine(replace(w, cache_depths=keep))
            ev.prefill()
            t0 = time.perf_counter()
            ev.prefill()
            torch.cuda.synchronize()
            pf_ms = (time.perf_counter() - t0) * 1e3
            fe = Runner(ev, args.steps, args.warmup).timed(w.tau_ent)
            tok, cl = ev.out_tokens.cpu().numpy(), ev.out_cl.cpu().numpy()
            both = (cl != 0) & (cl_full != 0)
            extra["kv_evict"]["keep_%d" % keep] = dict(
                tok_s=fe["tok_s"], ms_per_step=fe["ms_per_step"], committed_per_step=fe["committed_per_step"],
                loops=fe["loops"], prefill_ms=pf_ms, cache_bytes=plane * (D.kv_slots(keep) + 1),
                cache_bytes_full=plane * D.kv_slots(w.k_max),
                token_agreement=float((tok[both] == tok_full[both]).mean()) if both.any() else None)
            ev.close()
            del ev
        # the other workloads
        n2 = max(1, min(args.steps, 10))
        sec = argparse.Namespace(steps=n2, warmup=min(args.warmup, 3))
        for name in ("qwen3_1p7b", "qwen3_8b_long"):
            if name in args.configs:
                torch.cuda.empty_cache()
                fig, ex, _ = step_config(Engine, synth.workload(name), sec)
                ex.close()
                del ex
                extra[name] = fig
        if "readout" in args.configs:
            torch.cuda.empty_cache()
            extra["readout"] = {str(n): readout_config(Engine, n, sec) for n in synth.READOUT_ROWS}
    else:
        e.close()

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
                   "tau_ent": w.tau_ent, "tau_halt": w.tau_halt, "exit_b": w.exit_bias(),
                   "parallelism": "single GPU"},
        "roofline": head["roofline"],
        "loops": head["loops"],
        "loops_per_token": head["loops_per_token"],
        "mean_first_loop_lambda": head["mean_first_loop_lambda"],
        "committed_per_step": head["committed_per_step"],
        "prefill_ms": head["prefill_ms"],
        "tau_sweep": head.get("tau_sweep"),
        # per class: event-timed ms (the event pairs add a little time to short kernels, so the
        # fractions are lower bounds) with algorithmic bytes / flops and their roofline fractions
        "kernels": head["kernels"],
        "timing_pass_ms_per_step": head["timing_pass_ms_per_step"],
        **extra,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, w.tau_ent)
    kill_children()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
