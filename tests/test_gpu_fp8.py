"""GPU parity of fp8 (OCP E4M3) key/value storage -- the compressed depth buffers -- against the
fp64 oracle with the same storage format."""
from dataclasses import replace

import numpy as np
import pytest

from adaptive_looped_denoising_amd import synth
from oracle import alodlm_oracle as orc
from oracle import run as orun
from tests.parity import CAL_FACTOR, NS_HIDDEN, log, rel_rows
from tests.stepcheck import check_step

pytestmark = pytest.mark.gpu

MID_DIMS = synth.Dims(vocab=4096, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024, n_pre=2,
                      n_core=2, n_coda=2)


def _mid(**over):
    base = synth.Workload("mid_fp8", MID_DIMS, "bf16", batch=3, prefix=300, block=32, k_max=4, tau_ent=0.6,
                          tau_halt=0.6, seed=11, boost_lo=10.0, boost_hi=16.0, kv_dtype="fp8")
    return replace(base, **over)


def _engine(w, **kw):
    from adaptive_looped_denoising_amd.engine import Engine
    e = Engine(w, **kw)
    e.prefill()
    return e


def test_fp8_synthetic_cache_is_the_oracle_rounding_bit_for_bit(gpu_lib):
    """Synthetic K/V are float32 draws rounded once to E4M3 on the device; the oracle rounds the same
    draws with its own E4M3 rounding: every stored value must agree exactly (ties included)."""
    w = _mid(kv="synthetic", prefix=130, batch=2, short_frac=0.25, short_depth=2)
    e = _engine(w)
    W = orun.weights(w, names=[])
    av = synth.avail_depth(w)
    for b in range(w.batch):
        cache = orun.cache_for(w, W, b)
        for slot in range(w.dims.kv_slots(w.k_max)):
            gk, gv = e.read_kv(slot, b, 0, w.prefix)
            D = w.dims
            if D.n_pre <= slot < D.n_pre + D.n_core * w.k_max:  # materialised planes: depth min(plane, avail)
                c, dp = divmod(slot - D.n_pre, w.k_max)
                src = [D.n_pre + c * w.k_max + min(dp + 1, int(a)) - 1 for a in av[b]]
                ok = np.stack([cache[s][0][:, j] for j, s in enumerate(src)], axis=1)
                ov = np.stack([cache[s][1][:, j] for j, s in enumerate(src)], axis=1)
            else:
                ok, ov = cache[slot]
            assert np.array_equal(gk, ok) and np.array_equal(gv, ov), "seq %d slot %d" % (b, slot)


def _check_cache(e, w, b, n, ref, ref16):
    """fp8 cache rows against the oracle's fp8 cache: within the bf16 tolerance or CAL_FACTOR x the
    drift of the bf16 rounding-point oracle, at every depth (E4M3 keeps 3 fraction bits, so an fp8
    rounding that the two sides take on either side of a tie moves one element by one E4M3 step,
    which the bf16 figure alone does not cover; the drift of the fp8 rounding-point oracle does)."""
    worst = 0.0
    for slot in range(w.dims.kv_slots(w.k_max)):
        gk, gv = e.read_kv(slot, b, 0, n)
        for gi, g in enumerate((gk, gv)):
            o = np.asarray(ref[slot][gi])[:, :n].reshape(-1, w.dims.head_dim)
            o16 = np.asarray(ref16[slot][gi])[:, :n].reshape(-1, w.dims.head_dim)
            err = float(rel_rows(g.reshape(-1, w.dims.head_dim), o).max())
            tol = max(NS_HIDDEN["bf16"], CAL_FACTOR * float(rel_rows(o16, o).max()))
            assert err <= tol, "seq %d slot %d err %.3g > %.3g" % (b, slot, err, tol)
            worst = max(worst, err / tol)
    return worst


def test_mid_fp8_prefill_cache(gpu_lib):
    w = _mid(prefix=130, batch=2)
    e = _engine(w)
    W = orun.weights(w)
    ids = synth.prefix_ids(w)
    for b in range(w.batch):
        ref = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8")
        ref16 = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8", prec="bf16")
        log("seq %d worst/tol %.3f" % (b, _check_cache(e, w, b, w.prefix, ref, ref16)))


def _check_step(w, sample=None):
    e = _engine(w)
    ores, free, _ = check_step(w, e, sample=sample, name=w.name + " fp8 K/V")
    return e, ores, free


def test_mid_fp8_step_prefill_cache(gpu_lib):
    _check_step(_mid())


def test_mid_fp8_step_synthetic_cache_depth_fallback(gpu_lib):
    _check_step(_mid(kv="synthetic", short_frac=0.25, short_depth=2, tau_ent=0.0, tau_halt=2.0, prefix=700, batch=2))


def test_mid_fp8_outer_loop_and_append(gpu_lib):
    """Outer loop over fp8 storage, then the finished block appended (written in fp8)."""
    from tests.test_gpu_outer import _flagged
    w = _mid(prefix=130, batch=2, tau_ent=1.5, boost_lo=6.0, boost_hi=14.0)
    e = _engine(w, max_prefix=w.prefix + w.block)
    g = e.denoise_block(append=True)
    ores = orun.denoise_block(w)
    W = orun.weights(w)
    for r in ores:
        b = r["seq"]
        if not _flagged(w, r):
            assert np.array_equal(g["tokens"][b], r["tokens"]) and np.array_equal(g["commit_step"][b], r["commit_step"])
        ids = np.concatenate([synth.prefix_ids(w)[b], g["tokens"][b]])
        ref = orc.prefill_sequence(ids, W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8")
        ref16 = orc.prefill_sequence(ids, W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8", prec="bf16")
        log("seq %d grown cache worst/tol %.3f" % (b, _check_cache(e, w, b, w.prefix + w.block, ref, ref16)))


def test_mid_fp8_head_dim_64(gpu_lib):
    """fp8 K/V at hd 64: the conversion pass into the 64-wide working tile and its swizzle."""
    dims = replace(MID_DIMS, head_dim=64, n_q_heads=8, n_kv_heads=1)
    _check_step(replace(_mid(prefix=200, batch=2), dims=dims))
