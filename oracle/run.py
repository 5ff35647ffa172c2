"""Drives the oracle over a seeded synthetic workload (test infrastructure only).

Builds the oracle's inputs from the shared seeded generator and runs the
per-sequence oracle step; nothing here reads GPU results.
"""
from __future__ import annotations

from dataclasses import replace
from typing import Dict, List, Optional

import numpy as np

from adaptive_looped_denoising_amd import synth
from oracle import alodlm_oracle as orc


def weights(w: synth.Workload, names: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """Workload weights as float32 arrays holding the exact stored values."""
    return {k: synth.as_f32(v) for k, v in synth.host_weights(w, names).items()}


def kv_format(w: synth.Workload):
    """The oracle's K/V storage option for the workload: "fp8" or None (the model dtype)."""
    return "fp8" if w.kv_dtype == "fp8" else None


def keep_depths(w: synth.Workload) -> int:
    """Core depths the workload's cache keeps (depth eviction below k_max)."""
    return w.cache_depths or w.k_max


def avail_for(w: synth.Workload, av_b):
    """Available depths a step reads for one sequence: the supplied ones, clipped by eviction."""
    if not w.prefix:
        return None
    if keep_depths(w) == w.k_max:
        return av_b
    return orc.evict_depths({}, av_b, w.dims, w.k_max, keep_depths(w), w.prefix)[1]


def cache_for(w: synth.Workload, W, b: int, prefix_ids=None, progress=None, prec=None) -> Dict[int, tuple]:
    """Depth-aware prefix cache of sequence b: computed by the oracle's prefill, or the
    workload's synthetic K/V (with fp8 K/V: the float32 draws rounded by the oracle's E4M3);
    with depth eviction, the Core sets deeper than the kept depths are dropped."""
    if w.prefix == 0:
        return {}
    if w.kv == "synthetic":
        out = {}
        for slot in range(w.dims.kv_slots(w.k_max)):
            if kv_format(w) == "fp8":
                K, V = synth.synthetic_kv_seq(replace(w, dtype="fp32"), slot, b)
                out[slot] = (orc.round_fp8_e4m3(K), orc.round_fp8_e4m3(V))
            else:
                K, V = synth.synthetic_kv_seq(w, slot, b)
                out[slot] = (synth.as_f32(K), synth.as_f32(V))
    else:
        ids = synth.prefix_ids(w) if prefix_ids is None else prefix_ids
        out = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, progress=progress,
                                   prec=prec, kv=kv_format(w))
    if keep_depths(w) < w.k_max:
        out = orc.evict_depths(out, None, w.dims, w.k_max, keep_depths(w), w.prefix)[0]
    return out


def step(w: synth.Workload, W=None, seqs=None, k_loops: Optional[int] = None, teacher=None,
         record_hidden: bool = False, block_ids=None, boost=None, avail=None, caches=None,
         exit_b: Optional[float] = None, counter: Optional[list] = None, progress=None,
         prec=None, sample: Optional[dict] = None) -> List[dict]:
    """Oracle denoising step for the listed sequences of the workload (``prec`` as in
    alodlm_oracle.layer_forward; ``sample`` = {"seed", "step"} commits Gumbel-max draws)."""
    W = weights(w) if W is None else W
    seqs = range(w.batch) if seqs is None else seqs
    bids = synth.block_ids(w) if block_ids is None else block_ids
    btok, bval = synth.boosts(w) if boost is None else boost
    av = synth.avail_depth(w) if avail is None else avail
    pids = synth.prefix_ids(w) if (w.kv == "prefill" and w.prefix) else None
    out = []
    for b in seqs:
        cache = caches[b] if caches is not None else cache_for(w, W, b, pids, progress, prec)
        res = orc.denoise_step_sequence(
            bids[b], cache, avail_for(w, av[b] if av is not None else None), W, w.dims,
            k_max=w.k_max, k_loops=w.k_max if k_loops is None else k_loops, eps=w.rms_eps,
            theta=w.rope_theta, tau_ent=w.tau_ent, tau_halt=w.tau_halt, mask_id=w.mask_id,
            exit_b=w.exit_bias() if exit_b is None else exit_b, boost_tok=btok[b], boost_val=bval[b],
            teacher=None if teacher is None else teacher[b], record_hidden=record_hidden, counter=counter,
            progress=progress, prec=prec, sample=None if sample is None else dict(sample, seq=b), kv=kv_format(w))
        res["seq"] = b
        out.append(res)
    return out


def step_kwargs(w: synth.Workload, k_loops: Optional[int] = None, exit_b: Optional[float] = None) -> dict:
    """Keyword arguments of the oracle step for the workload's model and thresholds."""
    return dict(k_max=w.k_max, k_loops=w.k_max if k_loops is None else k_loops, eps=w.rms_eps,
                theta=w.rope_theta, tau_ent=w.tau_ent, tau_halt=w.tau_halt,
                exit_b=w.exit_bias() if exit_b is None else exit_b)


def denoise_block(w: synth.Workload, W=None, seqs=None, block_ids=None, boost=None, caches=None, avail=None,
                  sample: Optional[dict] = None, max_steps: Optional[int] = None, prec=None) -> List[dict]:
    """Oracle outer loop (steps until no mask) for the listed sequences of the workload
    (``sample`` = {"seed", "step0"})."""
    W = weights(w) if W is None else W
    seqs = range(w.batch) if seqs is None else seqs
    bids = synth.block_ids(w) if block_ids is None else block_ids
    btok, bval = synth.boosts(w) if boost is None else boost
    av = synth.avail_depth(w) if avail is None else avail
    pids = synth.prefix_ids(w) if (w.kv == "prefill" and w.prefix) else None
    out = []
    for b in seqs:
        cache = caches[b] if caches is not None else cache_for(w, W, b, pids, None, prec)
        res = orc.denoise_block_sequence(
            bids[b], cache, avail_for(w, av[b] if av is not None else None), W, w.dims, max_steps=max_steps,
            sample=None if sample is None else dict(sample, seq=b), mask_id=w.mask_id, boost_tok=btok[b],
            boost_val=bval[b], prec=prec, kv=kv_format(w), **step_kwargs(w))
        res["seq"] = b
        out.append(res)
    return out


def denoise_block_on_demand(w: synth.Workload, depth0: int, W=None, sample: Optional[dict] = None,
                            prec=None) -> dict:
    """Oracle outer loop over the whole batch with a depth-on-demand cache: every prefix built to
    depth0; after a step whose loop count over the batch exceeds the built depth, every cache is
    deepened to that loop count before the next step (``sample`` = {"seed", "step0"})."""
    W = weights(w) if W is None else W
    D = w.dims
    pids = synth.prefix_ids(w)
    btok, bval = synth.boosts(w)
    caches, states = {}, {}
    for b in range(w.batch):
        caches[b], states[b] = orc.prefill_sequence(pids[b], W, D, w.k_max, w.rms_eps, w.rope_theta, prec=prec,
                                                    depth=depth0, state=True, kv=kv_format(w))
    built = depth0
    ids = {b: np.asarray(synth.block_ids(w)[b], dtype=np.int64).copy() for b in range(w.batch)}
    commit_step = {b: np.zeros(w.block, dtype=np.int64) for b in range(w.batch)}
    commit_loop = {b: np.zeros(w.block, dtype=np.int64) for b in range(w.batch)}
    results, depths = [], []
    t = 0
    while any((ids[b] == w.mask_id).any() for b in range(w.batch)):
        t += 1
        loops_max = 0
        for b in range(w.batch):
            if not (ids[b] == w.mask_id).any():
                continue
            smp = None if sample is None else dict(seed=sample["seed"], step=sample["step0"] + t - 1, seq=b)
            res = orc.denoise_step_sequence(ids[b], caches[b], np.full(w.prefix, built), W, D, mask_id=w.mask_id,
                                            boost_tok=btok[b], boost_val=bval[b], prec=prec, sample=smp,
                                            kv=kv_format(w), **step_kwargs(w))
            newly = res["commit_loop"] != 0
            commit_step[b][newly] = t
            commit_loop[b][newly] = res["commit_loop"][newly]
            ids[b] = np.asarray(res["tokens"], dtype=np.int64).copy()
            loops_max = max(loops_max, res["loops"])
            results.append((t, b, res))
        if loops_max > built:
            for b in range(w.batch):
                caches[b], states[b] = orc.deepen_sequence(caches[b], states[b], W, D, w.k_max, w.rms_eps,
                                                           w.rope_theta, built, loops_max, prec=prec, kv=kv_format(w))
            built = loops_max
        depths.append(built)
    return dict(tokens=ids, commit_step=commit_step, commit_loop=commit_loop, steps=t, built_depth=built,
                depth_after_step=depths, results=results)


def teacher_from(results: List[dict]) -> Dict[int, dict]:
    """Teacher-forcing decisions (commit loops, tokens, stop loop) taken from oracle results."""
    return {r["seq"]: dict(commit_loop=r["commit_loop"], tokens=r["tokens"], stop_loop=r["loops"])
            for r in results}


def near_decisions(w: synth.Workload, res: dict, ent_tol: float = 1e-2, gap_tol: float = 1e-2,
                   halt_tol: float = 1e-2) -> List[str]:
    """Decisions of one oracle sequence that sit within the tolerances of a threshold:
    |H - tau_ent|, top-2 logit gap of a committed token, |mean a - tau_halt|, forced-commit
    entropy gap.  In sampling mode the gap that decides a committed token is the top-2 gap of
    z + g.  A GPU free run may legitimately differ from the oracle only there."""
    flags = []
    for rec in res["records"]:
        rows = rec["rows"]
        gap = rec.get("sgap", rec["gap"])
        if rows.size:
            d = np.abs(rec["H"][rows] - w.tau_ent)
            if (d < ent_tol).any():
                flags.append("entropy loop %d rows %s" % (rec["loop"], rows[d < ent_tol].tolist()))
        for i in rec["committed"]:
            if gap[i] < gap_tol:
                flags.append("token gap loop %d row %d" % (rec["loop"], i))
        if rec["n_unresolved"] and abs(rec["mean_a"] - w.tau_halt) < halt_tol:
            flags.append("halt loop %d" % rec["loop"])
    if res["forced"] >= 0:
        last = res["records"][-1]
        if res["forced_gap"] < ent_tol:
            flags.append("forced entropy gap")
        if last.get("sgap", last["gap"])[res["forced"]] < gap_tol:
            flags.append("forced token gap")
    return flags
