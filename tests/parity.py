"""Comparison helpers of the GPU step against the oracle (shared by the GPU tests, smoke and bench)."""
from __future__ import annotations

import sys
from typing import List

import numpy as np

from adaptive_looped_denoising_amd import synth
from oracle import run as orun

# Tolerances.  Hidden states / readout rows: row-wise relative L2 error.  Entropy: absolute nats.
# lambda and a: absolute; derived from the hidden-state bound through the ExitGate dot product
# (|d(w.r)| ~ weight_std * ||dr||, sigmoid slope <= 1/4).
TOL = {
    "fp32": dict(hidden=1e-4, H=1e-4, lam=1e-4, a=1e-4, lse=1e-4),
    "bf16": dict(hidden=2e-2, H=1e-2, lam=2e-2, a=2e-2, lse=2e-2),
}


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_rows(x: np.ndarray, ref: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(x - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-30)


def compare_records(w: synth.Workload, oracle_res: List[dict], gpu, check_hidden: bool = True,
                    seqs=None) -> dict:
    """Per-loop entropy, lambda, a, lse, argmax and Core output of the GPU step against the oracle
    (both must have taken the same decisions, e.g. in teacher-forced mode).  Returns worst errors."""
    tol = TOL[w.dtype]
    worst = dict(H=0.0, lam=0.0, a=0.0, lse=0.0, hidden=0.0, tok_mismatch=0)
    for res in oracle_res:
        b = res["seq"]
        for rec in res["records"]:
            s = rec["loop"] - 1
            rows = rec["rows"]
            gH = gpu.entropy[s, b]
            read = np.isfinite(gH)
            assert np.array_equal(np.nonzero(read)[0], rows), "seq %d loop %d: rows read out differ" % (b, s + 1)
            if rows.size:
                for key, g, o in (("H", gpu.entropy, rec["H"]), ("lam", gpu.lam, rec["lam"]),
                                  ("a", gpu.halt, rec["a"]), ("lse", gpu.lse, rec["lse"])):
                    err = np.abs(g[s, b, rows] - o[rows])
                    if key == "lse":
                        err = err / np.maximum(np.abs(o[rows]), 1.0)
                    worst[key] = max(worst[key], float(err.max()))
                    assert err.max() <= tol[key], "seq %d loop %d %s err %.3g > %.3g" % (
                        b, s + 1, key, err.max(), tol[key])
                mism = gpu.argmax[s, b, rows] != rec["tok"][rows]
                if mism.any():  # only allowed where the oracle's top-2 gap is within the flag tolerance
                    assert (rec["gap"][rows][mism] < 1e-2).all(), "seq %d loop %d argmax mismatch" % (b, s + 1)
                    worst["tok_mismatch"] += int(mism.sum())
            if check_hidden and gpu.hidden is not None and "h_tilde" in rec:
                e = rel_rows(gpu.hidden[s, b], rec["h_tilde"])
                worst["hidden"] = max(worst["hidden"], float(e.max()))
                assert e.max() <= tol["hidden"], "seq %d loop %d hidden rel err %.3g" % (b, s + 1, e.max())
    return worst


def compare_decisions(w: synth.Workload, oracle_res: List[dict], gpu) -> List[int]:
    """Free-run decisions must match exactly for every sequence the oracle does not flag as near
    a decision boundary.  Returns the flagged sequences."""
    flagged = []
    for res in oracle_res:
        b = res["seq"]
        flags = orun.near_decisions(w, res)
        if flags:
            log("seq %d near decision boundaries: %s" % (b, "; ".join(flags)))
            flagged.append(b)
            continue
        assert gpu.loops[b] == res["loops"], "seq %d loops %d vs oracle %d" % (b, gpu.loops[b], res["loops"])
        assert np.array_equal(gpu.commit_loop[b], res["commit_loop"]), "seq %d commit schedule %s vs %s" % (
            b, gpu.commit_loop[b], res["commit_loop"])
        assert np.array_equal(gpu.tokens[b], res["tokens"]), "seq %d tokens differ" % b
    return flagged
