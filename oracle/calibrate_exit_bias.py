"""Writes the ExitGate bias of each seeded workload (adaptive_looped_denoising_amd/exit_bias.json).

Test-infrastructure script: it calls only the oracle.  The bias is an input of the synthetic
workloads, set so that the mean first-loop halting probability over the block rows of the seeded
inputs is the value the method pages report for a trained model: the mean first-pass halting
probability of 0.417 (tokendh.com explainer of the ALoDLM paper; summary page "ALoDLM: Adaptively
Looped Diffusion Language Models", section Results, Fig. 4 right), taken as 0.42.

Procedure (per workload): the oracle runs loop 1 of the step with bias 0 and records every block
row's readout state r (loop 1 comes before any halting decision, so r does not depend on the
bias); t = w_g . r is the ExitGate logit without bias; the bias b solves
mean_rows sigmoid(t + b) = target by bisection in float64 and is stored rounded to float32 (the
precision both the oracle and the library take it in).  The readout microbench's rows are given,
so there t = w_g . row directly.

Usage: python -m oracle.calibrate_exit_bias [workload ...]   (default: every workload)
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from adaptive_looped_denoising_amd import synth  # noqa: E402
from oracle import run  # noqa: E402

OUT = os.path.join(ROOT, "adaptive_looped_denoising_amd", "exit_bias.json")
TARGET = 0.42
# sequences whose loop-1 readout the bias is solved on (the whole batch where the oracle's prefill
# of it takes minutes, else a stated sample)
SEQS = {"tiny": None, "qwen3_1p7b": None, "qwen3_8b": None, "qwen3_8b_long": [0, 1, 2, 3]}


def solve(t: np.ndarray, target: float = TARGET) -> float:
    """b with mean(sigmoid(t + b)) = target (the mean is increasing in b)."""
    lo, hi = -60.0, 60.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if np.mean(1.0 / (1.0 + np.exp(-(t + mid)))) < target:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def first_loop_logits(w: synth.Workload, seqs) -> np.ndarray:
    W = run.weights(w)
    res = run.step(w, W=W, seqs=seqs, k_loops=1, record_hidden=True, exit_b=0.0,
                   progress=lambda m: print("  " + m, flush=True) if m.endswith("layer 0") else None)
    return np.concatenate([rec["r"] @ np.asarray(W["exit_w"], dtype=np.float64) for r in res
                           for rec in r["records"][:1]])


def readout_logits(n_rows: int) -> np.ndarray:
    rows = synth.as_f32(synth.readout_rows(n_rows))
    w = synth.readout_workload(n_rows)
    wg = synth.as_f32(synth.host_weights(w, ["exit_w"])["exit_w"])
    return rows.astype(np.float64) @ wg.astype(np.float64)


def main(names):
    table = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            table = json.load(f).get("bias", {})
    for name in names:
        t0 = time.time()
        if name.startswith("readout_"):
            t = readout_logits(int(name.split("_")[1]))
            sample = "all %d readout rows" % t.size
        else:
            w = synth.workload(name)
            seqs = SEQS.get(name)
            t = first_loop_logits(w, seqs)
            sample = "loop-1 readout of %s (%d rows)" % ("every sequence" if seqs is None else "sequences %s" % seqs,
                                                         t.size)
        b = float(np.float32(solve(t)))
        lam = 1.0 / (1.0 + np.exp(-(t + b)))
        wl = synth.readout_workload(int(name.split("_")[1])) if name.startswith("readout_") else synth.workload(name)
        table[name] = dict(exit_b=b, mean_first_loop_lambda=float(lam.mean()), logit_mean=float(t.mean()),
                           logit_std=float(t.std()), sample=sample, inputs=synth.bias_fingerprint(wl))
        print("%s: b = %.6f, mean lambda %.4f over %s (%.0f s)" % (name, b, lam.mean(), sample, time.time() - t0),
              flush=True)
        with open(OUT, "w") as f:
            json.dump(dict(target=TARGET, written_by="oracle/calibrate_exit_bias.py",
                           source="mean first-pass halting probability 0.417: tokendh.com explainer; summary page "
                                  "'ALoDLM: Adaptively Looped Diffusion Language Models', Results, Fig. 4 right",
                           bias=table), f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or ["tiny"] + ["readout_%d" % n for n in synth.READOUT_ROWS] +
         ["qwen3_1p7b", "qwen3_8b_long", "qwen3_8b"])
