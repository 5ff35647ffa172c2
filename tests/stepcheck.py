"""One GPU denoising step against the oracle: free run compared position by position, records
compared while both runs agree, then a teacher-forced run compared loop by loop (shared by the
GPU step tests and the smoke check)."""
from __future__ import annotations

import numpy as np

from oracle import run as orun
from tests.parity import (KEYS, agreed_loops, calibrated, compare_decisions, compare_records, literal_tolerances,
                          log, loop_depth, rel_rows, report, tolerances)

# tolerances that never fail: for comparisons that are measured and reported only
UNBOUNDED = dict(hidden=np.inf, lse=np.inf, lam=np.inf, a=np.inf, H=np.inf, ent_flag=np.inf, gap=np.inf, halt=np.inf)


def oracle_drift(exact, rounded) -> dict:
    """Worst deviation of the oracle's bf16 rounding-point run from the exact run (same decisions),
    over every record of every sequence: entropy, lambda, a, lse (relative) and the Core output."""
    out = dict(hidden=0.0, H=0.0, lam=0.0, a=0.0, lse=0.0)
    for res, res16 in zip(exact, rounded):
        for a, c in zip(res["records"], res16["records"]):
            rows = a["rows"]
            if rows.size:
                for k in ("H", "lam", "a"):
                    out[k] = max(out[k], float(np.abs(a[k][rows] - c[k][rows]).max()))
                out["lse"] = max(out["lse"], float((np.abs(a["lse"][rows] - c["lse"][rows]) /
                                                    np.maximum(np.abs(a["lse"][rows]), 1.0)).max()))
            if "h_tilde" in a and "h_tilde" in c:
                out["hidden"] = max(out["hidden"], float(rel_rows(c["h_tilde"], a["h_tilde"]).max()))
    return out


def check_step(w, e, W=None, seqs=None, caches=None, k_loops=None, block_ids=None, sample=None, name="",
               teacher_check=True):
    """Runs the engine's step free and teacher-forced and the oracle on sequences ``seqs``.
    Returns (oracle results, free GPU result, decision summary per sequence)."""
    W = orun.weights(w) if W is None else W
    K = w.k_max if k_loops is None else k_loops
    log("case %s dtype=%s B=%d P=%d L=%d K=%d tau=%.3g q=%.3g sample=%s seqs=%s" % (
        name or w.name, w.dtype, w.batch, w.prefix, w.block, K, w.tau_ent, w.tau_halt, sample,
        "all" if seqs is None else list(seqs)))
    free = e.step(k_loops=K, records=True, hidden=True, block_ids=block_ids, sample=sample)
    ores = orun.step(w, W=W, seqs=seqs, k_loops=K, record_hidden=True, block_ids=block_ids, caches=caches,
                     sample=sample)
    deep = calibrated(w, loop_depth(w, max([r["loops"] for r in ores] + [1])))
    o16 = None
    if deep:   # the oracle's own bf16 drift on this input and these decisions
        o16 = orun.step(w, W=W, seqs=seqs, k_loops=K, record_hidden=True, block_ids=block_ids, caches=caches,
                        prec="bf16", teacher=orun.teacher_from(ores), sample=sample)
    tols = tolerances(w, ores, o16)
    assert free.n_committed == int((free.commit_loop != 0).sum())
    dec = compare_decisions(w, ores, free, tols)
    worst_free = compare_records(w, ores, free, tols, upto=agreed_loops(ores, dec))
    log("free run: worst errors %s; decisions %s" % (worst_free, dec))
    worst_tf = worst_rp = None
    if teacher_check:
        teacher = orun.teacher_from(ores)
        for b in range(w.batch):   # sequences the oracle did not run keep the GPU's own decisions
            if b not in teacher:
                teacher[b] = dict(commit_loop=free.commit_loop[b], tokens=free.tokens[b], stop_loop=free.loops[b])
        tf = e.step(k_loops=K, records=True, hidden=True, teacher=teacher, block_ids=block_ids, sample=sample)
        worst_tf = compare_records(w, ores, tf, tols)
        for r in ores:
            b = r["seq"]
            assert np.array_equal(tf.commit_loop[b], r["commit_loop"]) and np.array_equal(tf.tokens[b], r["tokens"])
            assert tf.loops[b] == r["loops"]
        log("teacher-forced: worst errors %s" % worst_tf)
        if o16 is not None:
            # the same teacher-forced GPU run against the oracle's bf16 rounding-point run on the
            # same decisions: measured and reported, bounded only through the exact comparison
            worst_rp = compare_records(w, o16, tf, lambda b, loop: UNBOUNDED)
            log("teacher-forced vs the rounding-point oracle: worst errors %s" % worst_rp)
            drift = oracle_drift(ores, o16)
            log("rounding-point oracle vs the exact oracle: worst %s" % drift)
    worst = {k: max(worst_free.get(k, 0.0), (worst_tf or {}).get(k, 0.0)) for k in ("hidden", "H", "lam", "a", "lse")}
    depth = max(loop_depth(w, r["loops"]) for r in ores) if any(r["loops"] for r in ores) else 0
    report(name or w.name, "%s %s B=%d P=%d L=%d K=%d" % (w.name, w.dtype, w.batch, w.prefix, w.block, K), worst,
           literal_tolerances(w.dtype),
           dict(layer_calls=depth, tier="calibrated" if deep else "literal",
                positions_compared_free=sum(d["compared"] for d in dec.values()),
                sequences_diverged=[b for b, d in dec.items() if d["diverged"] is not None],
                entropy_commits=int(sum(int((r["commit_loop"] > 0).sum()) for r in ores)),
                vs_rounding_points=None if worst_rp is None else {k: worst_rp[k] for k in KEYS},
                rounding_points_vs_exact=None if worst_rp is None else drift))
    return ores, free, dec
