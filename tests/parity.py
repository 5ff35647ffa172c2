"""Comparison helpers of the GPU step against the oracle (shared by the GPU tests, smoke and bench)."""
from __future__ import annotations

import sys
from typing import List

import numpy as np

from adaptive_looped_denoising_amd import synth
from oracle import run as orun

# Tolerances.  Hidden states / readout rows: row-wise relative L2 error.  Entropy: absolute nats.
#
# fp32 mode: fixed (1e-4).  bf16 mode: the pipeline rounds its GEMM / attention inputs to bf16
# (unit roundoff 2^-9) at about five points per layer call, so its deviation from exact
# arithmetic is a sum of independent per-layer rounding noises and grows like sqrt(depth):
#   hidden(n) = 2e-2 * max(1, sqrt(n / 16))            n = layer calls the rows went through
# (2e-2 through 16 layer calls, the depth of the small workloads).  The readout quantities follow
# from it: a relative error e of a unit-RMS readout row r moves the logits z = W r by about
# e * sigma_z (sigma_z^2 = weight_std^2 * d, the logit variance) and the entropy by about
# e * Var(z) (dH/dz_i = -p_i (z_i - E_p z)), the ExitGate logit by about e * weight_std * sqrt(d)
# (slope of the sigmoid <= 1/4); each bound below takes twice that.
BF16_BASE, BF16_DEPTH = 2e-2, 16


def tol_hidden(dtype: str, n: int) -> float:
    if dtype == "fp32":
        return 1e-4
    return BF16_BASE * max(1.0, (n / BF16_DEPTH) ** 0.5)


def tolerances(w: synth.Workload, n: int) -> dict:
    """Tolerances for quantities computed after n layer calls."""
    if w.dtype == "fp32":
        return dict(hidden=1e-4, H=1e-4, lam=1e-4, a=1e-4, lse=1e-4, gap=1e-2, halt=1e-4)
    e = tol_hidden("bf16", n)
    var_z = w.weight_std ** 2 * w.dims.d_model
    return dict(hidden=e, H=max(1e-2, 2 * var_z * e), lam=max(2e-2, 0.5 * w.weight_std * w.dims.d_model ** 0.5 * e),
                a=max(2e-2, 0.5 * w.weight_std * w.dims.d_model ** 0.5 * e),
                lse=max(2e-2, 2 * var_z * e), gap=max(1e-2, 2 * var_z ** 0.5 * e),
                halt=max(1e-2, 0.5 * w.weight_std * w.dims.d_model ** 0.5 * e))


def loop_depth(w: synth.Workload, loop: int) -> int:
    """Layer calls a block row has gone through when it is read out at `loop`."""
    D = w.dims
    return D.n_pre + loop * (D.n_core + D.n_coda)


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


CAL_FACTOR = 3.0


def calibrated_tolerances(w: synth.Workload, exact: List[dict], rounded: List[dict]) -> dict:
    """Per (sequence, loop) tolerances: the depth model above, or CAL_FACTOR times the deviation of
    the bf16 rounding-point oracle from the exact oracle on the same decisions, whichever is
    larger.  That deviation is the drift any pipeline rounding at those points incurs on this
    input; both runs are the oracle's, nothing comes from the GPU."""
    out = {}
    for re_, rr in zip(exact, rounded):
        for a, c in zip(re_["records"], rr["records"]):
            t = dict(tolerances(w, loop_depth(w, a["loop"])))
            rows = a["rows"]
            if rows.size:
                t["H"] = max(t["H"], CAL_FACTOR * float(np.abs(a["H"][rows] - c["H"][rows]).max()))
                t["lam"] = max(t["lam"], CAL_FACTOR * float(np.abs(a["lam"][rows] - c["lam"][rows]).max()))
                t["a"] = max(t["a"], CAL_FACTOR * float(np.abs(a["a"][rows] - c["a"][rows]).max()))
                t["halt"] = max(t["halt"], t["a"])
                t["lse"] = max(t["lse"], CAL_FACTOR * float(
                    (np.abs(a["lse"][rows] - c["lse"][rows]) / np.maximum(np.abs(a["lse"][rows]), 1.0)).max()))
            if "h_tilde" in a and "h_tilde" in c:
                t["hidden"] = max(t["hidden"], CAL_FACTOR * float(rel_rows(a["h_tilde"], c["h_tilde"]).max()))
            t["gap"] = max(t["gap"], 2 * (w.weight_std ** 2 * w.dims.d_model) ** 0.5 * t["hidden"])
            out[(re_["seq"], a["loop"])] = t
    return out


def compare_records(w: synth.Workload, oracle_res: List[dict], gpu, check_hidden: bool = True,
                    seqs=None, tols: dict = None) -> dict:
    """Per-loop entropy, lambda, a, lse, argmax and Core output of the GPU step against the oracle
    (both must have taken the same decisions, e.g. in teacher-forced mode).  Returns worst errors.
    ``tols`` (optional): per (sequence, loop) tolerances from calibrated_tolerances."""
    worst = dict(H=0.0, lam=0.0, a=0.0, lse=0.0, hidden=0.0, tok_mismatch=0)
    for res in oracle_res:
        b = res["seq"]
        for rec in res["records"]:
            s = rec["loop"] - 1
            tol = tols[(b, rec["loop"])] if tols else tolerances(w, loop_depth(w, rec["loop"]))
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
                    assert (rec["gap"][rows][mism] < tol["gap"]).all(), "seq %d loop %d argmax mismatch" % (b, s + 1)
                    worst["tok_mismatch"] += int(mism.sum())
                if "stok" in rec and getattr(gpu, "sampled", None) is not None:
                    mism = gpu.sampled[s, b, rows] != rec["stok"][rows]
                    if mism.any():  # the draw may differ only where the top-2 gap of z + g is within tolerance
                        assert (rec["sgap"][rows][mism] < tol["gap"]).all(), "seq %d loop %d draw mismatch" % (
                            b, s + 1)
                        worst["tok_mismatch"] += int(mism.sum())
            if check_hidden and gpu.hidden is not None and "h_tilde" in rec:
                e = rel_rows(gpu.hidden[s, b], rec["h_tilde"])
                worst["hidden"] = max(worst["hidden"], float(e.max()))
                assert e.max() <= tol["hidden"], "seq %d loop %d hidden rel err %.3g" % (b, s + 1, e.max())
    return worst


def compare_decisions(w: synth.Workload, oracle_res: List[dict], gpu, tols: dict = None) -> List[int]:
    """Free-run decisions must match exactly for every sequence the oracle does not flag as near
    a decision boundary.  Returns the flagged sequences."""
    flagged = []
    for res in oracle_res:
        b = res["seq"]
        if res["loops"] == 0:  # nothing masked: no decision was taken
            flags = []
        else:
            t = tols[(b, res["loops"])] if tols else tolerances(w, loop_depth(w, res["loops"]))
            flags = orun.near_decisions(w, res, ent_tol=t["H"], gap_tol=t["gap"], halt_tol=t["halt"])
        if flags:
            log("seq %d near decision boundaries: %s" % (b, "; ".join(flags)))
            flagged.append(b)
            continue
        assert gpu.loops[b] == res["loops"], "seq %d loops %d vs oracle %d" % (b, gpu.loops[b], res["loops"])
        assert np.array_equal(gpu.commit_loop[b], res["commit_loop"]), "seq %d commit schedule %s vs %s" % (
            b, gpu.commit_loop[b], res["commit_loop"])
        assert np.array_equal(gpu.tokens[b], res["tokens"]), "seq %d tokens differ" % b
    return flagged
