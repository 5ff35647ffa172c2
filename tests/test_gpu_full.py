"""GPU parity at the full workload sizes (1.7B shape, 8B shape, 8B long context), in the launch
configuration the benchmark times, against the fp64 oracle:

* prefill: causal attention makes the first positions of the depth-aware cache depend on those
  positions only, so the oracle recomputes them exactly from the token ids;
* step: sequences are independent (per-sequence halting), so the oracle recomputes whole
  sequences of the batch -- over the cache the library's prefill built (1.7B shape, as the
  workload states it) or over the seeded synthetic cache (8B shapes);
* fp32 mode at the same shapes: the literal fp32 tolerances at full depth;
* determinism: the matrix-core step run twice gives the same bits.
"""
import gc
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from adaptive_looped_denoising_amd import synth
from oracle import alodlm_oracle as orc
from oracle import run as orun
from tests.parity import cache_tolerance, log, rel_rows, report, literal_tolerances
from tests.stepcheck import check_step

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_W_CACHE = {}


def _oracle_weights(w):
    key = (w.dims, w.seed, w.dtype)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        gc.collect()
        log("generating host weights for %s (%s)" % (w.name, w.dtype))
        _W_CACHE[key] = orun.weights(w)
    return _W_CACHE[key]


def _engine(w, **kw):
    from adaptive_looped_denoising_amd.engine import Engine
    gc.collect()
    torch.cuda.empty_cache()
    e = Engine(w, **kw)
    e.prefill()
    return e


def _effective(w, b, n_pos, cache):
    """The oracle cache as the GPU stores it after the prefill: Core depth slots hold every position
    at depth min(depth, available depth), the depth a step at that loop reads."""
    D = w.dims
    av = synth.avail_depth(w)[b, :n_pos].astype(int)
    out = {}
    for slot in range(D.kv_slots(w.k_max)):
        if D.n_pre <= slot < D.n_pre + D.n_core * w.k_max:
            c, dp = divmod(slot - D.n_pre, w.k_max)
            src = D.n_pre + c * w.k_max + np.maximum(1, np.minimum(dp + 1, av)) - 1
        else:
            src = np.full(n_pos, slot)
        K = np.stack([np.asarray(cache[int(s)][0])[:, j] for j, s in enumerate(src)], axis=1)
        V = np.stack([np.asarray(cache[int(s)][1])[:, j] for j, s in enumerate(src)], axis=1)
        out[slot] = (K, V)
    return out


def _layer_depth(w, slot):
    """Layer calls the prefix has gone through when it produces the K/V of a cache slot."""
    D = w.dims
    if slot < D.n_pre:
        return slot + 1
    if slot < D.n_pre + D.n_core * w.k_max:
        c, dpt = divmod(slot - D.n_pre, w.k_max)
        return D.n_pre + dpt * D.n_core + c + 1
    return D.n_pre + w.k_max * D.n_core + (slot - D.n_pre - D.n_core * w.k_max) + 1


def _check_prefill_prefix(w, n_pos, seqs):
    """GPU prefill over the full prefix vs the oracle's prefill of the first n_pos tokens, slot by
    slot (relative error of each position's K and V rows): within the literal tolerance, or
    CAL_FACTOR times the drift of the oracle's own bf16 rounding-point prefill from the exact one
    where that is larger (tests.parity.cache_tolerance)."""
    e = _engine(w)
    W = _oracle_weights(w)
    ids = synth.prefix_ids(w)
    hd = w.dims.head_dim
    for b in seqs:
        log("oracle prefill of the first %d positions of sequence %d" % (n_pos, b))
        kw = dict(dims=w.dims, k_max=w.k_max, eps=w.rms_eps, theta=w.rope_theta)
        c64 = _effective(w, b, n_pos, orc.prefill_sequence(ids[b][:n_pos], W, **kw))
        c16 = _effective(w, b, n_pos, orc.prefill_sequence(ids[b][:n_pos], W, prec="bf16", **kw)) \
            if w.dtype == "bf16" else c64
        worst = 0.0
        for slot in range(w.dims.kv_slots(w.k_max)):
            gk, gv = e.read_kv(slot, b, 0, n_pos)
            err = drift = 0.0
            for g, o64, o16 in zip((gk, gv), c64[slot], c16[slot]):
                o64 = np.asarray(o64).reshape(-1, hd)
                err = max(err, float(rel_rows(g.reshape(-1, hd), o64).max()))
                drift = max(drift, float(rel_rows(np.asarray(o16).reshape(-1, hd), o64).max()))
            tol = cache_tolerance(w.dtype, drift)
            assert err <= tol, "seq %d slot %d (depth %d): err %.3g > %.3g" % (b, slot, _layer_depth(w, slot), err, tol)
            worst = max(worst, err)
        log("seq %d worst slot error %.4g (literal %.0e)" % (b, worst, literal_tolerances(w.dtype)["hidden"]))
    e.close()


def _check(w, seqs, prefill_cache=False, sample=None, name="", **ekw):
    """Step parity on sequences ``seqs``: over the synthetic cache, or (prefill_cache) over the
    cache the library's prefill built, which the oracle rebuilds from the token ids."""
    e = _engine(w, **ekw)
    W = _oracle_weights(w)
    caches = None if prefill_cache else {b: orun.cache_for(w, W, b) for b in seqs}
    ores, free, dec = check_step(w, e, W=W, seqs=seqs, caches=caches, sample=sample, name=name)
    log("GPU commits per sequence %s, loops %s" % ((free.commit_loop != 0).sum(axis=1).tolist(), free.loops.tolist()))
    return e, ores, free, dec


# --------------------------------------------------------------------------- 1.7B shape
def test_qwen3_1p7b_prefill_first_positions(gpu_lib):
    _check_prefill_prefix(synth.workload("qwen3_1p7b"), 16, [0])


def test_qwen3_1p7b_step_on_prefill_cache(gpu_lib):
    """The 1.7B-shape workload as stated: the step over the depth-aware cache alodlm_prefill_kv
    built from the 512 prefix tokens, compared end to end (the oracle runs the whole prefill)."""
    w = synth.workload("qwen3_1p7b")
    e, _, _, _ = _check(w, [0], prefill_cache=True, name="qwen3_1p7b prefill cache")
    e.close()


def test_qwen3_1p7b_fp32_step_on_prefill_cache(gpu_lib):
    """fp32 mode at the 1.7B shape over the prefill-built cache: the literal fp32 tolerances
    (hidden rows and logits 1e-4, entropies 1e-2 nats, decisions flagged at 1e-2) at full depth."""
    w = synth.workload("qwen3_1p7b", dtype="fp32", tau_ent=0.9, boost_lo=10.0, boost_hi=20.0)
    e, ores, _, dec = _check(w, [0], prefill_cache=True, name="qwen3_1p7b fp32 prefill cache")
    assert all(d["diverged"] is None for d in dec.values())
    e.close()


def test_qwen3_1p7b_pages_split_without_prelude_and_coda(gpu_lib):
    """The pages' own 1.7B split: no Prelude, no Coda, the Core loops over all 28 layers (4 loops:
    112 layer calls), bf16 over a synthetic cache; then the same split in fp32 mode with entropy
    commits, at the literal tolerances."""
    dims = replace(synth.QWEN3_1P7B_DIMS, n_pre=0, n_core=28, n_coda=0)
    w = replace(synth.workload("qwen3_1p7b", kv="synthetic", tau_ent=-1.0, tau_halt=2.0), dims=dims,
                name="qwen3_1p7b_0_28_0")
    e, ores, _, _ = _check(w, [0], name="1.7B split 0/28/0")
    calls, loops = e.stats()
    assert loops == 4 and calls == 4 * 28
    e.close()
    wf = replace(w, dtype="fp32", tau_ent=0.9, tau_halt=0.5, boost_lo=10.0, boost_hi=20.0)
    e, _, _, _ = _check(wf, [0], name="1.7B split 0/28/0 fp32")
    e.close()


# --------------------------------------------------------------------------- 8B shape
def test_qwen3_8b_prefill_first_positions(gpu_lib):
    _check_prefill_prefix(synth.workload("qwen3_8b"), 8, [0, 5])


@pytest.mark.skipif(os.environ.get("ALODLM_LONG_TESTS") != "1",
                    reason="about 150 s of oracle prefill on the host; run with ALODLM_LONG_TESTS=1")
def test_qwen3_8b_step_on_prefill_cache(gpu_lib):
    """The 8B-shape workload as benchmarked: the step over the depth-aware cache alodlm_prefill_kv
    built from the 8 x 1024 prefix tokens, one sequence compared end to end (the oracle runs that
    sequence's whole prefill, 84 layer calls over 1024 positions, exactly and at the bf16 rounding
    points).  Opt-in: the oracle's two fp64 prefills of 1024 positions take about 150 s."""
    w = synth.workload("qwen3_8b")
    e, _, _, _ = _check(w, [0], prefill_cache=True, name="qwen3_8b prefill cache")
    e.close()


def test_qwen3_8b_step_sampled_sequences(gpu_lib):
    w = synth.workload("qwen3_8b", kv="synthetic")
    e, _, _, _ = _check(w, [0, 7], name="qwen3_8b")
    # structural pin: with entropy commits and halting off the 8B split runs 10 + 4 x (16 + 10) layers
    e.step(tau_ent=-1.0, tau_halt=2.0)
    calls, loops = e.stats()
    assert loops == 4 and calls == 114
    e.close()


def test_qwen3_8b_step_with_entropy_commits(gpu_lib):
    """Planted boosts strong enough that easy rows commit by entropy at the 8B vocabulary size;
    decisions compared position by position on two sequences."""
    w = synth.workload("qwen3_8b", kv="synthetic", boost_lo=10.0, boost_hi=20.0, tau_ent=0.9)
    e, ores, _, dec = _check(w, [2, 6], name="qwen3_8b entropy commits")
    assert sum(int((r["commit_loop"] > 0).sum()) for r in ores) > 0
    # at least one sequence with entropy commits had its whole commit schedule compared free-running
    assert any(dec[r["seq"]]["diverged"] is None and (r["commit_loop"] > 0).any() for r in ores)
    e.close()


def test_qwen3_8b_fp32_step_with_entropy_commits(gpu_lib):
    """fp32 mode at the 8B dimensions (d 4096, 32/8 heads, FFN 12288, vocabulary 151936, 10/16/10
    layers, 1024 cached positions) with entropy commits: the literal fp32 tolerances at full depth,
    decisions position by position.  Two sequences: the fp32 path's attention is the plain vector
    kernel (one wave per query row and head), too slow for the eight of the bf16 workload."""
    w = synth.workload("qwen3_8b", kv="synthetic", dtype="fp32", boost_lo=10.0, boost_hi=20.0, tau_ent=0.9,
                       batch=2)
    e, ores, _, dec = _check(w, [1], name="qwen3_8b fp32 entropy commits (batch 2)")
    assert sum(int((r["commit_loop"] > 0).sum()) for r in ores) > 0
    assert all(d["diverged"] is None for d in dec.values())
    e.close()


def test_qwen3_8b_sampled_commits(gpu_lib):
    """Sampled commits at the 8B vocabulary (151936 Gumbel-max candidates per row) in the benchmark's
    launch configuration: draws, commit schedule and tokens against the oracle's own generator."""
    w = synth.workload("qwen3_8b", kv="synthetic", boost_lo=10.0, boost_hi=20.0, tau_ent=0.9)
    e, ores, free, _ = _check(w, [3], sample=dict(seed=0xA11CE5EED, step=17), name="qwen3_8b sampled")
    assert sum(int((r["commit_loop"] > 0).sum()) for r in ores) > 0
    assert free.sampled is not None and (free.sampled[0] >= 0).sum() > 0
    e.close()


def test_qwen3_8b_fp32_sampled_commits(gpu_lib):
    """Sampled commits in fp32 mode at the 8B dimensions (151936 Gumbel-max candidates per row,
    10/16/10 layers): draws, commit schedule and tokens against the oracle's own generator at the
    literal fp32 tolerances, no decision differing."""
    w = synth.workload("qwen3_8b", kv="synthetic", dtype="fp32", boost_lo=10.0, boost_hi=20.0, tau_ent=0.9,
                       batch=2)
    e, ores, free, dec = _check(w, [0], sample=dict(seed=0x5EED0FF5, step=3),
                                name="qwen3_8b fp32 sampled (batch 2)")
    assert sum(int((r["commit_loop"] > 0).sum()) for r in ores) > 0
    assert free.sampled is not None and (free.sampled[0] >= 0).sum() > 0
    assert all(d["diverged"] is None for d in dec.values())
    e.close()


def test_qwen3_8b_fp8_kv_step(gpu_lib):
    """fp8 (E4M3) keys and values at the 8B shape over the synthetic cache."""
    w = synth.workload("qwen3_8b", kv="synthetic", kv_dtype="fp8")
    e, _, _, _ = _check(w, [1], name="qwen3_8b fp8 K/V")
    e.close()


def test_qwen3_8b_step_is_deterministic(gpu_lib):
    """The matrix-core step (split-K and split-KV partials merged in fixed order, no atomics in any
    sum) run twice: every output, record and hidden row bit for bit."""
    w = synth.workload("qwen3_8b", kv="synthetic", boost_lo=10.0, boost_hi=20.0, tau_ent=0.9)
    e = _engine(w)
    a = e.step(records=True, hidden=True)
    b = e.step(records=True, hidden=True)
    for k in ("tokens", "commit_loop", "loops", "entropy", "lam", "halt", "lse", "argmax", "hidden"):
        x, y = getattr(a, k), getattr(b, k)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k
    log("8B step twice: identical bits (%d commits, loops %s)" % (a.n_committed, a.loops.tolist()))
    e.close()


# --------------------------------------------------------------------------- long context
def test_qwen3_8b_long_context_step(gpu_lib):
    """The long-context workload as benchmarked (batch 32, 8192 cached positions, K_max 6), one
    sequence against the oracle; then the whole step twice, bit for bit (its GEMMs run single-pass
    on the 256 x 256 tile and its attention without key splits: a different set of kernels from the
    8B step's)."""
    w = synth.workload("qwen3_8b_long")
    e, _, _, _ = _check(w, [5], name="qwen3_8b_long")
    a = e.step(records=True, hidden=True)
    b = e.step(records=True, hidden=True)
    for k in ("tokens", "commit_loop", "loops", "entropy", "lam", "halt", "lse", "argmax", "hidden"):
        x, y = getattr(a, k), getattr(b, k)
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), k
    log("long-context step twice: identical bits (%d commits, loops %s)" % (a.n_committed, a.loops.tolist()))
    e.close()


def test_qwen3_8b_long_context_fp32_step(gpu_lib):
    """fp32 mode at the long-context shape (8192 cached positions, a quarter of them cached at
    depths 1..3 only, K_max 6, tau_halt 0.9) with entropy commits: the literal fp32 tolerances at
    full depth (up to 166 layer calls), decisions position by position.  One sequence: the fp32
    path's attention is the plain vector kernel."""
    w = synth.workload("qwen3_8b_long", dtype="fp32", batch=1, boost_lo=10.0, boost_hi=20.0, tau_ent=0.9)
    e, ores, _, dec = _check(w, [0], name="qwen3_8b_long fp32 entropy commits (batch 1)")
    assert sum(int((r["commit_loop"] > 0).sum()) for r in ores) > 0
    assert all(d["diverged"] is None for d in dec.values())
    e.close()
