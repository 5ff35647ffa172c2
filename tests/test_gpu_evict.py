"""GPU parity of depth eviction -- a cache that keeps Core depths 1..D only, deeper loops reading the
deepest kept depth -- against the fp64 oracle's evicted cache."""
from dataclasses import replace

import numpy as np
import pytest

from adaptive_looped_denoising_amd import synth
from oracle import alodlm_oracle as orc
from oracle import run as orun
from tests.parity import cache_tolerance, log, rel_rows
from tests.stepcheck import check_step

pytestmark = pytest.mark.gpu

MID_DIMS = synth.Dims(vocab=4096, d_model=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1024, n_pre=2,
                      n_core=2, n_coda=2)


def _mid(**over):
    base = synth.Workload("mid_evict", MID_DIMS, "bf16", batch=2, prefix=130, block=32, k_max=4, tau_ent=0.6,
                          tau_halt=0.6, seed=11, boost_lo=10.0, boost_hi=16.0, cache_depths=2)
    return replace(base, **over)


def _engine(w, **kw):
    from adaptive_looped_denoising_amd.engine import Engine
    e = Engine(w, **kw)
    e.prefill()
    return e


def _stored(w, cache, avail):
    """The evicted oracle cache as the library stores it: stored slot -> (K, V, layer calls), Core
    plane p (1..D) holding every position j at depth min(p, avail_j)."""
    D = w.dims
    keep = orun.keep_depths(w)
    av = np.asarray(avail, dtype=np.int64)
    out = []
    for li in range(D.n_layers):
        core = D.n_pre <= li < D.n_pre + D.n_core
        if not core:
            K, V = cache[orc.kv_slot(D, w.k_max, li)]
            calls = li + 1 if li < D.n_pre else li + 1 + (w.k_max - 1) * D.n_core
            out.append((np.asarray(K), np.asarray(V), calls))
            continue
        for p in range(1, keep + 1):
            dep = np.minimum(p, av)
            K0 = np.asarray(cache[orc.kv_slot(D, w.k_max, li, 1)][0])
            K, V = np.empty(K0.shape), np.empty(K0.shape)
            for d in np.unique(dep):
                sel = dep == d
                Kd, Vd = cache[orc.kv_slot(D, w.k_max, li, int(d))]
                K[:, sel], V[:, sel] = np.asarray(Kd)[:, sel], np.asarray(Vd)[:, sel]
            out.append((K, V, D.n_pre + (p - 1) * D.n_core + (li - D.n_pre) + 1))
    return out


def _check_cache(e, w, b, j0, n, ref, ref16=None, exact=False):
    """Every stored slot of sequence b, rows j0 .. j0+n-1, against ``ref`` (from _stored): bit-exact,
    or within tests.parity.cache_tolerance (the drift taken from the rounding-point oracle ``ref16``)."""
    assert len(ref) == e.kv_slots == w.dims.kv_slots(orun.keep_depths(w))
    worst = 0.0
    for slot, (K, V, calls) in enumerate(ref):
        gk, gv = e.read_kv(slot, b, j0, n)
        for gi, (g, o) in enumerate(((gk, K), (gv, V))):
            o = o[:, j0:j0 + n]
            if exact:
                assert np.array_equal(g, o), "seq %d slot %d" % (b, slot)
                continue
            err = float(rel_rows(g.reshape(-1, w.dims.head_dim), o.reshape(-1, w.dims.head_dim)).max())
            drift = 0.0
            if w.dtype == "bf16":
                o16 = ref16[slot][gi][:, j0:j0 + n]
                drift = float(rel_rows(o16.reshape(-1, w.dims.head_dim), o.reshape(-1, w.dims.head_dim)).max())
            tol = cache_tolerance(w.dtype, drift)
            assert err <= tol, "seq %d slot %d rows %d..%d error %.3g > %.3g" % (b, slot, j0, j0 + n, err, tol)
            worst = max(worst, err / tol)
    return worst


def _check_step_fp32(w, e, caches=None, avail=None):
    ores = orun.step(w, record_hidden=True, caches=caches, avail=avail)
    g = e.step(records=True, hidden=True)
    for r in ores:
        b = r["seq"]
        assert g.loops[b] == r["loops"] and np.array_equal(g.commit_loop[b], r["commit_loop"])
        assert np.array_equal(g.tokens[b], r["tokens"])
        for rec in r["records"]:
            assert rel_rows(g.hidden[rec["loop"] - 1, b], rec["h_tilde"]).max() < 1e-4
    return ores


@pytest.mark.parametrize("keep", [1, 2])
def test_tiny_fp32_evicted_prefill_and_step(gpu_lib, keep):
    """Prefill with depths above `keep` evicted (their passes run in the scratch plane): the kept
    sets equal the oracle's full prefill, the Coda set included; a step reads loops > keep at keep."""
    w = synth.workload("tiny", batch=2, boost_lo=8.0, boost_hi=14.0, tau_ent=0.3, tau_halt=0.9,
                       short_frac=0.25, short_depth=1, cache_depths=keep)
    e = _engine(w)
    W = orun.weights(w)
    av = synth.avail_depth(w)
    for b in range(w.batch):
        ref = _stored(w, orun.cache_for(w, W, b), orun.avail_for(w, av[b]))
        log("seq %d cache worst/tol %.3f" % (b, _check_cache(e, w, b, 0, w.prefix, ref)))
    ores = _check_step_fp32(w, e)
    log("loops %s" % [r["loops"] for r in ores])
    assert max(r["loops"] for r in ores) > keep


def test_tiny_fp32_evicted_extend_twice_then_step(gpu_lib):
    """Two blocks appended to a cache keeping two depths: the appended positions' deeper passes read
    the cached positions at depth <= 2 (from the kept plane, the earlier appended rows included)."""
    w = synth.workload("tiny", batch=2, boost_lo=8.0, boost_hi=14.0, short_frac=0.25, short_depth=1,
                       cache_depths=2)
    e = _engine(w, max_prefix=w.prefix + 24)
    new = np.random.default_rng(3).integers(0, w.dims.vocab, size=(w.batch, 24)).astype(np.int32)
    e.extend(new[:, :10])
    e.extend(new[:, 10:])
    W = orun.weights(w)
    av = synth.avail_depth(w)
    kw = dict(dims=w.dims, k_max=w.k_max, eps=w.rms_eps, theta=w.rope_theta, keep=2)
    caches, avs = {}, []
    for b in range(w.batch):
        c, a = orun.cache_for(w, W, b), orun.avail_for(w, av[b])
        c, a = orc.extend_sequence(c, a, new[b, :10], W, **kw)
        c, a = orc.extend_sequence(c, a, new[b, 10:], W, **kw)
        caches[b] = c
        avs.append(a)
        log("seq %d cache worst/tol %.3f" % (b, _check_cache(e, w, b, 0, w.prefix + 24, _stored(w, c, a))))
    _check_step_fp32(w, e, caches=caches, avail=np.stack(avs))


def test_tiny_fp32_evicted_outer_loop_and_append(gpu_lib):
    from tests.test_gpu_outer import _check_block
    w = synth.workload("tiny", batch=2, boost_lo=8.0, boost_hi=14.0, tau_ent=0.8, cache_depths=1)
    e = _engine(w, max_prefix=w.prefix + w.block)
    g = e.denoise_block(append=True)
    ores = orun.denoise_block(w)
    _check_block(w, e, ores, g)
    W = orun.weights(w)
    for b in range(w.batch):
        c, a = orc.extend_sequence(orun.cache_for(w, W, b), orun.avail_for(w, synth.avail_depth(w)[b]),
                                   g["tokens"][b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, keep=1)
        _check_cache(e, w, b, w.prefix, w.block, _stored(w, c, a))


def test_mid_bf16_evicted_synthetic_cache_is_exact(gpu_lib):
    """Synthetic K/V: each kept slot holds the draws of its slot in the full layout, materialised at
    the clipped depths, bit for bit."""
    w = _mid(kv="synthetic", short_frac=0.25, short_depth=1, prefix=200)
    e = _engine(w)
    W = orun.weights(w, names=[])
    av = synth.avail_depth(w)
    for b in range(w.batch):
        _check_cache(e, w, b, 0, w.prefix, _stored(w, orun.cache_for(w, W, b), orun.avail_for(w, av[b])),
                     exact=True)


def _check_step_bf16(w):
    e = _engine(w)
    ores, _, _ = check_step(w, e, name=w.name + " evicted")
    return e, ores


def test_mid_bf16_evicted_prefill_cache_and_step(gpu_lib):
    w = _mid(tau_ent=0.0, tau_halt=2.0)
    e, ores = _check_step_bf16(w)
    assert max(r["loops"] for r in ores) == w.k_max
    W = orun.weights(w)
    ids = synth.prefix_ids(w)
    for b in range(w.batch):
        a = orun.avail_for(w, synth.avail_depth(w)[b])
        full = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
        full16 = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, prec="bf16")
        ref = _stored(w, orc.evict_depths(full, None, w.dims, w.k_max, 2, w.prefix)[0], a)
        ref16 = [(K, V) for K, V, _ in _stored(w, orc.evict_depths(full16, None, w.dims, w.k_max, 2, w.prefix)[0], a)]
        log("seq %d cache worst/tol %.3f" % (b, _check_cache(e, w, b, 0, w.prefix, ref, ref16)))


def test_mid_bf16_evicted_extend(gpu_lib):
    w = _mid(kv="synthetic", short_frac=0.25, short_depth=1, prefix=200)
    e = _engine(w, max_prefix=260)
    new = np.random.default_rng(4).integers(0, w.dims.vocab, size=(w.batch, 40)).astype(np.int32)
    e.extend(new)
    W = orun.weights(w)
    av = synth.avail_depth(w)
    kw = dict(dims=w.dims, k_max=w.k_max, eps=w.rms_eps, theta=w.rope_theta, keep=2)
    for b in range(w.batch):
        c, a = orun.cache_for(w, W, b), orun.avail_for(w, av[b])
        ref_c, ref_a = orc.extend_sequence(c, a, new[b], W, **kw)
        ref16_c, _ = orc.extend_sequence(c, a, new[b], W, prec="bf16", **kw)
        ref = _stored(w, ref_c, ref_a)
        ref16 = [(K, V) for K, V, _ in _stored(w, ref16_c, ref_a)]
        log("seq %d new rows worst/tol %.3f" % (b, _check_cache(e, w, b, w.prefix, 40, ref, ref16)))


def test_mid_fp8_evicted_step_and_cache(gpu_lib):
    """Both compressions of the depth buffers at once: fp8 K/V in a cache keeping two depths."""
    w = _mid(kv_dtype="fp8", prefix=130, tau_ent=0.0, tau_halt=2.0)
    e, ores = _check_step_bf16(w)
    assert max(r["loops"] for r in ores) == w.k_max
    W = orun.weights(w)
    ids = synth.prefix_ids(w)
    for b in range(w.batch):
        a = orun.avail_for(w, synth.avail_depth(w)[b])
        full = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8")
        full16 = orc.prefill_sequence(ids[b], W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8", prec="bf16")
        ref = _stored(w, orc.evict_depths(full, None, w.dims, w.k_max, 2, w.prefix)[0], a)
        ref16 = [(K, V) for K, V, _ in _stored(w, orc.evict_depths(full16, None, w.dims, w.k_max, 2, w.prefix)[0], a)]
        log("seq %d cache worst/tol %.3f" % (b, _check_cache(e, w, b, 0, w.prefix, ref, ref16)))
