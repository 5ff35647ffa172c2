"""Pins of the oracle to facts it does not compute itself: closed forms, textbook identities,
brute force on tiny inputs, the structural counts printed on the method pages, and an
independently written straight-line forward.  CPU only."""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch

from adaptive_looped_denoising_amd import synth
from oracle import alodlm_oracle as orc
from oracle import run

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tiny(**over):
    return synth.workload("tiny", **over)


def _rand_weights(w, seed=0):
    """Random weights with non-unit gains (so gains are exercised), float64."""
    rng = np.random.default_rng(seed)
    W = {}
    for s in synth.weight_specs(w):
        if "const" in s:
            W[s["name"]] = 1.0 + 0.1 * rng.standard_normal(s["shape"])
        else:
            W[s["name"]] = 0.05 * rng.standard_normal(s["shape"])
    return W


# --------------------------------------------------------------------------- generator
def test_philox_known_answers():
    for v in _golden("philox4x32_10_kat.json")["vectors"]:
        out = synth.philox4x32_10([int(x, 16) for x in v["ctr"]], [int(x, 16) for x in v["key"]])
        assert [int(x) for x in out] == [int(x, 16) for x in v["out"]]


def test_generator_ranges_and_layouts():
    w = _tiny()
    ids = synth.prefix_ids(w)
    assert ids.shape == (1, 32) and ids.min() >= 0 and ids.max() < w.dims.vocab
    tok, val = synth.boosts(w)
    easy = tok >= 0
    assert easy.sum() == w.n_easy == 10
    assert (val[easy] >= 4).all() and (val[easy] < 10).all() and (val[~easy] == 0).all()
    assert tok.max() <= w.dims.vocab - 2
    # element ranges are the same numbers whichever slice is asked for
    full = synth.ih4((1000,), 7, 99, 0.5, "bf16")
    part = synth.ih4((100,), 7, 99, 0.5, "bf16", start=450)
    assert np.array_equal(full[450:550], part)
    w4 = synth.workload("qwen3_8b_long")
    w4s = replace(w4, batch=2, prefix=64)
    av = synth.avail_depth(w4s)
    assert (np.sort(np.unique(av)) == [3, 6]).all() and ((av == 3).sum(axis=1) == 16).all()


# --------------------------------------------------------------------------- layer primitives
def test_rmsnorm_of_constant_vector_is_gain():
    g = np.linspace(0.5, 2.0, 64)
    for c in (3.0, -0.25, 1e3):
        np.testing.assert_allclose(orc.rms_norm(np.full(64, c), g, 0.0), np.sign(c) * g, rtol=1e-14)


def test_rope_identity_norm_and_relative_position():
    rng = np.random.default_rng(1)
    hd = 32
    x = rng.standard_normal((3, hd))
    np.testing.assert_allclose(orc.rope(x, np.zeros(3), 1e6), x, rtol=0, atol=0)
    y = orc.rope(x, np.array([5, 77, 1000]), 1e4)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    q, k = rng.standard_normal(hd), rng.standard_normal(hd)
    dots = []
    for m, n in ((10, 3), (107, 100), (7, 0)):
        qm = orc.rope(q[None], np.array([m]), 1e4)[0]
        kn = orc.rope(k[None], np.array([n]), 1e4)[0]
        dots.append(qm @ kn)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)
    # rotate-half pairing: a unit vector on coordinate 0 turns into (cos, ..., sin at hd/2)
    e0 = np.zeros((1, hd)); e0[0, 0] = 1.0
    r = orc.rope(e0, np.array([2]), 1e6)[0]
    assert r[0] == pytest.approx(math.cos(2.0)) and r[hd // 2] == pytest.approx(math.sin(2.0))


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 5, 8))
    k = rng.standard_normal((2, 7, 8))
    v = rng.standard_normal((2, 7, 8))
    # GQA with group 2 equals MHA over duplicated kv heads [0, 0, 1, 1]
    gqa = orc.attention(q, k, v)
    mha = orc.attention(q, k[[0, 0, 1, 1]], v[[0, 0, 1, 1]])
    np.testing.assert_allclose(gqa, mha, rtol=1e-14)
    # identical keys give the mean of the values
    kk = np.repeat(k[:, :1], 7, axis=1)
    np.testing.assert_allclose(orc.attention(q, kk, v)[0], np.broadcast_to(v[0].mean(0), (5, 8)), rtol=1e-12)
    # one visible key returns its value
    allowed = np.zeros((5, 7), dtype=bool); allowed[:, 3] = True
    np.testing.assert_allclose(orc.attention(q, k, v, allowed)[1], np.broadcast_to(v[0, 3], (5, 8)), rtol=1e-12)


def test_silu_values():
    assert orc.silu(0.0) == 0.0
    assert orc.silu(1.0) == pytest.approx(1.0 / (1.0 + math.exp(-1.0)), rel=1e-15)
    assert orc.silu(-40.0) == pytest.approx(-40.0 * math.exp(-40.0), rel=1e-9)


# --------------------------------------------------------------------------- heads
@pytest.mark.parametrize("V,lnV", [(512, 6.238325), (151936, 11.931215)])
def test_uniform_readout_entropy_is_log_vocab(V, lnV):
    r = np.ones((3, 16))
    H, tok, lse, gap = orc.readout(r, np.zeros((V, 16)))
    np.testing.assert_allclose(H, math.log(V), rtol=1e-12)
    assert abs(H[0] - lnV) < 1e-6
    assert (tok == 0).all() and (gap == 0).all()
    np.testing.assert_allclose(lse, math.log(V), rtol=1e-12)


@pytest.mark.parametrize("beta", [0.0, 1.5, 4.0, 10.0, 20.0])
def test_two_level_entropy_closed_form(beta):
    V = 512
    H, tok, _, _ = orc.readout(np.ones((1, 4)), np.zeros((V, 4)), [37], [beta])
    e = math.exp(beta)
    expect = math.log(e + V - 1) - beta * e / (e + V - 1)
    assert H[0] == pytest.approx(expect, rel=1e-12, abs=1e-13)
    assert tok[0] == (37 if beta > 0 else 0)


def test_readout_brute_force_tiny_vocab():
    rng = np.random.default_rng(3)
    for _ in range(20):
        V, d = int(rng.integers(2, 9)), int(rng.integers(1, 5))
        Wl = rng.standard_normal((V, d))
        r = rng.standard_normal((4, d))
        bt = rng.integers(-1, V, size=4)
        bv = rng.uniform(0, 3, size=4)
        H, tok, lse, _ = orc.readout(r, Wl, bt, bv)
        for i in range(4):
            z = [sum(Wl[t][j] * r[i][j] for j in range(d)) + (bv[i] if t == bt[i] else 0.0) for t in range(V)]
            Z = sum(math.exp(x) for x in z)
            ps = [math.exp(x) / Z for x in z]
            assert H[i] == pytest.approx(-sum(p * math.log(p) for p in ps), rel=1e-10, abs=1e-12)
            assert lse[i] == pytest.approx(math.log(Z), rel=1e-12)
            assert tok[i] == max(range(V), key=lambda t: (z[t], -t))


def test_argmax_ties_go_to_lowest_id():
    Wl = np.zeros((6, 2)); Wl[2] = [1, 0]; Wl[4] = [1, 0]
    _, tok, _, gap = orc.readout(np.array([[1.0, 0.0]]), Wl)
    assert tok[0] == 2 and gap[0] == 0


def test_exit_gate_sigmoid():
    lam = orc.exit_gate(np.zeros((2, 8)), np.zeros(8), math.log(0.42 / 0.58))
    np.testing.assert_allclose(lam, 0.42, rtol=1e-14)
    lam = orc.exit_gate(np.ones((1, 4)), np.array([1.0, -2.0, 0.5, 0.0]), 0.25)
    assert lam[0] == pytest.approx(1.0 / (1.0 + math.exp(0.25)), rel=1e-14)


def test_online_entropy_merge_equals_two_pass():
    """The streaming (max, S, T) merge a vocabulary-tiled readout uses reproduces H and lse."""
    rng = np.random.default_rng(4)
    z = rng.standard_normal(1000) * 3
    H_ref, _, lse_ref, _ = orc.readout(np.ones((1, 1)), z[:, None])
    for tile in (1, 7, 64, 333, 1000):
        M, S, T = -np.inf, 0.0, 0.0
        for o in range(0, z.size, tile):
            t = z[o:o + tile]
            m2 = t.max(); e = np.exp(t - m2); S2 = e.sum(); T2 = ((t - m2) * e).sum()
            Mn = max(M, m2)
            e1 = math.exp(M - Mn) if S else 0.0
            e2 = math.exp(m2 - Mn)
            T = ((T + (M - Mn) * S) * e1 if S else 0.0) + (T2 + (m2 - Mn) * S2) * e2
            S = S * e1 + S2 * e2
            M = Mn
        assert math.log(S) - T / S == pytest.approx(H_ref[0], rel=1e-12)
        assert M + math.log(S) == pytest.approx(lse_ref[0], rel=1e-12)


# --------------------------------------------------------------------------- cache structure
def test_kv_slot_count_matches_page():
    g = _golden("page_constants.json")
    d8 = synth.QWEN3_8B_DIMS
    assert (d8.n_pre, d8.n_pre + d8.n_core, d8.n_layers) == (10, 26, 36)
    assert tuple(g["layer_split_8b"]["value"]["core"]) == (10, 26)
    K = g["k_loops"]["value"]
    n_slots = d8.kv_slots(K)
    assert n_slots == g["kv_buffers_8b_k4"]["value"] == 84
    assert n_slots == d8.n_layers + (K - 1) * d8.n_core      # L + (K - 1) m
    assert d8.kv_slots(1) == g["kv_buffers_8b_k4"]["autoregressive_value"]
    slots = {orc.kv_slot(d8, K, l, dp) for l in range(36) for dp in range(1, K + 1)}
    assert slots == set(range(84))
    assert d8.kv_slots(6) == 116


def test_prefill_builds_every_slot_and_is_causal():
    w = _tiny()
    W = run.weights(w)
    ids = synth.prefix_ids(w)[0]
    cache = orc.prefill_sequence(ids, W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
    assert sorted(cache) == list(range(w.dims.kv_slots(w.k_max)))
    # causal: the cache of the first 10 positions does not depend on later tokens
    short = orc.prefill_sequence(ids[:10], W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
    for s in cache:
        np.testing.assert_allclose(cache[s][0][:, :10], short[s][0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(cache[s][1][:, :10], short[s][1], rtol=1e-12, atol=1e-14)


def test_depth_select_reads_min_of_loop_and_available_depth():
    d = synth.TINY_DIMS
    K, P = 4, 9
    cache = {}
    for l in range(d.n_layers):
        core = d.n_pre <= l < d.n_pre + d.n_core
        for dp in range(1, (K if core else 1) + 1):
            s = orc.kv_slot(d, K, l, dp)
            cache[s] = (np.full((d.n_kv_heads, P, 4), float(dp)), np.full((d.n_kv_heads, P, 4), 10.0 * dp + s))
    avail = np.array([1, 2, 3, 4, 4, 3, 2, 1, 4])
    for loop in range(1, K + 1):
        for l in range(d.n_pre, d.n_pre + d.n_core):
            Kc, Vc = orc.context_for(cache, d, K, l, loop, avail)
            expect = np.minimum(loop, avail)
            assert (Kc[0, :, 0] == expect).all()
            c = l - d.n_pre
            assert (Vc[1, :, 2] == 10.0 * expect + d.n_pre + c * K + expect - 1).all()
        Kp, _ = orc.context_for(cache, d, K, 0, loop, avail)
        assert (Kp == 1.0).all()


def test_layer_call_count_matches_page():
    g = _golden("page_constants.json")
    dims = replace(synth.QWEN3_8B_DIMS, vocab=64, d_model=16, n_q_heads=2, n_kv_heads=1, head_dim=8, ffn=16)
    w = replace(_tiny(), dims=dims, prefix=0, block=4, k_max=4, tau_ent=-1.0, tau_halt=2.0)
    calls = []
    res = run.step(w, counter=calls)
    assert res[0]["loops"] == 4
    assert len(calls) == g["layer_calls_8b_k4"]["value"] == 114
    assert 4 * dims.n_layers == g["layer_calls_8b_k4"]["full_stack_value"]


# --------------------------------------------------------------------------- step-level pins
def _torch_bf16(t):
    """torch's own rounding to bfloat16 (through float32, as a float32 pipeline stores it)."""
    return torch.from_numpy(np.ascontiguousarray(t, dtype=np.float64)).to(torch.float32).to(
        torch.bfloat16).to(torch.float64).numpy()


def _straight_line_readout(w, W, prefix, block, bf16=False):
    """Independent forward of [prefix ; block] through the whole stack in one pass: prefix rows
    attend causally, block rows attend to everything.  Returns the block rows' readout rows
    (final RMSNorm of the last layer's output) and their logits.  ``bf16``: values are rounded to
    bfloat16 (by torch) at the rounding points a bf16 pipeline has -- the normalised projection
    inputs, q and k after RoPE, v, the unnormalised attention probabilities that multiply v, the
    attention output, the SwiGLU output and the readout rows feeding the LM head; the residual
    stream, the softmax normaliser and the readout rows themselves stay exact."""
    D = w.dims
    Hq, Hkv, hd, F = D.n_q_heads, D.n_kv_heads, D.head_dim, D.ffn
    ids = np.concatenate([prefix, block])
    n, P = ids.size, prefix.size
    pos = np.arange(n, dtype=np.float64)
    x = np.array(W["embed"], dtype=np.float64)[ids]
    vis = np.tril(np.ones((n, n), dtype=bool))
    vis[P:, :] = True

    def norm(t, g):
        return t * (1.0 / np.sqrt((t ** 2).sum(-1, keepdims=True) / t.shape[-1] + w.rms_eps)) * g

    half = hd // 2
    freq = np.exp(-np.log(w.rope_theta) * np.arange(0, hd, 2) / hd)
    cos, sin = np.cos(np.outer(pos, freq)), np.sin(np.outer(pos, freq))

    def rot(t):  # t [n][H][hd]
        a, b = t[..., :half], t[..., half:]
        return np.concatenate([a * cos[:, None] - b * sin[:, None], a * sin[:, None] + b * cos[:, None]], -1)

    rb = _torch_bf16 if bf16 else (lambda t: t)
    for l in range(D.n_layers):
        g = lambda k: np.array(W["layers.%d.%s" % (l, k)], dtype=np.float64)
        t = rb(norm(x, g("attn_norm")))
        wq, wk, wv = np.split(g("wqkv"), [Hq * hd, (Hq + Hkv) * hd])
        q = rb(rot(norm(np.einsum("nd,od->no", t, wq).reshape(n, Hq, hd), g("q_norm"))))
        k = rb(rot(norm(np.einsum("nd,od->no", t, wk).reshape(n, Hkv, hd), g("k_norm"))))
        v = rb(np.einsum("nd,od->no", t, wv).reshape(n, Hkv, hd))
        k = np.repeat(k, Hq // Hkv, axis=1)
        v = np.repeat(v, Hq // Hkv, axis=1)
        sc = np.einsum("qhe,khe->hqk", q, k) / np.sqrt(hd)
        sc[:, ~vis] = -np.inf
        pr = np.exp(sc - sc.max(-1, keepdims=True))
        o = np.einsum("hqk,khe->qhe", rb(pr), v) / pr.sum(-1).transpose(1, 0)[:, :, None]
        o = rb(o.reshape(n, Hq * hd))
        x = x + o @ g("wo").T
        t = rb(norm(x, g("ffn_norm")))
        gate, up = np.split(t @ g("w_gate_up").T, 2, axis=1)
        x = x + rb(gate * (1.0 / (1.0 + np.exp(-gate))) * up) @ g("w_down").T
    r = norm(x[P:], np.array(W["final_norm"], dtype=np.float64))
    return r, rb(r) @ np.array(W["lm_head"], dtype=np.float64).T


def test_all_commit_reduces_to_one_fixed_depth_pass():
    """tau_ent >= ln V commits every masked row at loop 1: the tokens are the argmax of a plain
    fixed-depth stack (here with a one-deep cache, where the stack and the loop coincide)."""
    _all_commit_case((1, 2, 1))


def test_all_commit_reduction_without_prelude_and_coda():
    """The same reduction for a split whose Core is the whole stack (the pages' 1.7B layout)."""
    _all_commit_case((0, 4, 0))


def _all_commit_case(split):
    w = _tiny(k_max=1, tau_ent=math.log(512) + 1.0)
    w = replace(w, dims=replace(w.dims, n_pre=split[0], n_core=split[1], n_coda=split[2]))
    W = _rand_weights(w, seed=5)
    pre = synth.prefix_ids(w)[0]
    blk = synth.block_ids(w)[0].copy()
    blk[[1, 4]] = [17, 300]   # two rows already decoded
    res = run.step(w, W=W, block_ids=blk[None], boost=(np.full((1, 16), -1), np.zeros((1, 16))),
                   record_hidden=True)
    r_ref, z_ref = _straight_line_readout(w, W, pre, blk)
    expect = z_ref.argmax(axis=1)
    masked = blk == w.mask_id
    assert res[0]["loops"] == 1
    # the readout rows agree to rounding, and so do the entropies of the masked rows
    rec = res[0]["records"][0]
    np.testing.assert_allclose(rec["r"], r_ref, rtol=1e-10, atol=1e-12)
    p = np.exp(z_ref - z_ref.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(rec["H"][masked], -(p * np.log(p)).sum(axis=1)[masked], rtol=1e-10)
    assert (res[0]["commit_loop"][masked] == 1).all() and (res[0]["commit_loop"][~masked] == 0).all()
    assert np.array_equal(res[0]["tokens"][masked], expect[masked])
    assert np.array_equal(res[0]["tokens"][~masked], blk[~masked])


@pytest.mark.parametrize("gqa", [False, True])
def test_bf16_rounding_points_match_an_independent_forward(gqa):
    """The oracle's bf16 rounding-point mode (the drift model of a bf16 pipeline) rounds exactly at
    the documented points: with every masked row committing at loop 1 it equals the straight-line
    forward above rounded by torch at those points -- readout rows and entropies to fp64 rounding.
    A rounding point too many or too few moves them by bf16 noise (about 1e-3), far beyond."""
    w = _tiny(k_max=1, tau_ent=math.log(512) + 1.0)
    if not gqa:
        w = replace(w, dims=replace(w.dims, n_kv_heads=4))
    W = _rand_weights(w, seed=15)
    pre = synth.prefix_ids(w)[0]
    blk = synth.block_ids(w)[0].copy()
    blk[[2, 9]] = [41, 250]
    nob = (np.full((1, 16), -1), np.zeros((1, 16)))
    res = run.step(w, W=W, block_ids=blk[None], boost=nob, record_hidden=True, prec="bf16")
    exact = run.step(w, W=W, block_ids=blk[None], boost=nob, record_hidden=True)
    r_ref, z_ref = _straight_line_readout(w, W, pre, blk, bf16=True)
    rec = res[0]["records"][0]
    np.testing.assert_allclose(rec["r"], r_ref, rtol=1e-10, atol=1e-12)
    p = np.exp(z_ref - z_ref.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    masked = blk == w.mask_id
    np.testing.assert_allclose(rec["H"][masked], -(p * np.log(p)).sum(axis=1)[masked], rtol=1e-10)
    # and the rounding is real: the exact oracle differs by bf16 noise
    rel = np.linalg.norm(exact[0]["records"][0]["r"] - rec["r"], axis=1) / np.linalg.norm(rec["r"], axis=1)
    assert 1e-4 < rel.max() < 2e-2


@pytest.mark.parametrize("split", [(1, 2, 1), (0, 3, 0)])
def test_looping_equals_unrolling(split):
    """K loops of the shared Core equal one pass of a stack with the Core unrolled K times; also for
    the pages' 1.7B-style split without Prelude and Coda (the Core loops over the whole stack)."""
    K = 3
    w = _tiny(k_max=K, tau_ent=-1.0, tau_halt=2.0)
    w = replace(w, dims=replace(w.dims, n_pre=split[0], n_core=split[1], n_coda=split[2]))
    W = _rand_weights(w, seed=6)
    D = w.dims
    Du = replace(D, n_core=D.n_core * K)
    wu = replace(w, dims=Du, k_max=1)
    Wu = {k: v for k, v in W.items() if not k.startswith("layers.")}
    src = list(range(D.n_pre)) + [D.n_pre + c for _ in range(K) for c in range(D.n_core)] + \
        [D.n_pre + D.n_core + c for c in range(D.n_coda)]
    for lu, l in enumerate(src):
        for key in ("attn_norm", "wqkv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate_up", "w_down"):
            Wu["layers.%d.%s" % (lu, key)] = W["layers.%d.%s" % (l, key)]
    looped = run.step(w, W=W, record_hidden=True)[0]
    unrolled = run.step(wu, W=Wu, record_hidden=True)[0]
    assert looped["loops"] == K and unrolled["loops"] == 1
    a, b = looped["records"][-1], unrolled["records"][0]
    np.testing.assert_allclose(a["h_tilde"], b["h_tilde"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(a["H"], b["H"], rtol=1e-11)
    assert np.array_equal(a["tok"], b["tok"])


def test_uniform_depth_when_nothing_commits_and_halting_is_off():
    w = _tiny(tau_ent=0.0, tau_halt=1.5)
    res = run.step(w, record_hidden=True)[0]
    assert res["loops"] == w.k_max
    for rec in res["records"]:
        assert rec["committed"].size == 0
        assert (rec["H"][rec["rows"]] > 0).all()
    last = res["records"][-1]
    i = int(np.argmin(last["H"]))
    assert res["forced"] == i and res["commit_loop"][i] == -w.k_max and res["tokens"][i] == last["tok"][i]
    assert (np.delete(res["commit_loop"], i) == 0).all()


def test_uniform_readout_forces_lowest_position():
    w = _tiny(tau_ent=0.3)
    W = run.weights(w)
    W["lm_head"] = np.zeros_like(W["lm_head"])
    res = run.step(w, W=W, boost=(np.full((1, 16), -1), np.zeros((1, 16))))[0]
    for rec in res["records"]:
        np.testing.assert_allclose(rec["H"], math.log(512), rtol=1e-12)
    assert res["forced"] == 0 and res["tokens"][0] == 0 and res["commit_loop"][0] == -res["loops"]


def test_entropy_equal_to_threshold_commits():
    """Commit iff H <= tau (inclusive): with a uniform readout every row's entropy is the same
    value, and a threshold equal to it commits every masked row at loop 1."""
    w = _tiny()
    W = run.weights(w)
    W["lm_head"] = np.zeros_like(W["lm_head"])
    H0 = float(orc.readout(np.zeros((1, w.dims.d_model)), W["lm_head"])[0][0])
    res = run.step(replace(w, tau_ent=H0), W=W, boost=(np.full((1, 16), -1), np.zeros((1, 16))))[0]
    assert res["loops"] == 1 and (res["commit_loop"] == 1).all() and res["forced"] == -1
    assert (res["tokens"] == 0).all()


@pytest.mark.parametrize("lam,tau_halt,s_star", [(0.42, 0.5, 2), (0.42, 0.9, 5), (0.42, 0.3, 1), (0.2, 0.5, 4),
                                                 (0.5, 0.75, 2)])
def test_halting_closed_form(lam, tau_halt, s_star):
    K = 6
    w = _tiny(k_max=K, tau_ent=-1.0, tau_halt=tau_halt)
    W = run.weights(w)
    W["exit_w"] = np.zeros_like(W["exit_w"])
    res = run.step(w, W=W, exit_b=math.log(lam / (1 - lam)))[0]
    expect = min(K, math.ceil(math.log(1 - tau_halt) / math.log(1 - lam)))
    assert expect == s_star
    assert res["loops"] == s_star
    for rec in res["records"]:
        np.testing.assert_allclose(rec["a"], 1 - (1 - lam) ** rec["loop"], rtol=1e-12)


def test_halting_mean_is_over_unresolved_rows_only():
    """The stop rule averages a over the positions still unresolved: rows decoded before the step
    keep a = 0 and do not hold the sequence in the loop (the closed form over U still gives 2)."""
    lam, K = 0.42, 6
    w = _tiny(k_max=K, tau_ent=-1.0, tau_halt=0.5)
    W = run.weights(w)
    W["exit_w"] = np.zeros_like(W["exit_w"])
    blk = synth.block_ids(w)[0].copy()
    blk[:8] = np.arange(5, 13)
    res = run.step(w, W=W, block_ids=blk[None], exit_b=math.log(lam / (1 - lam)))[0]
    assert res["loops"] == 2
    last = res["records"][-1]
    assert (last["a"][:8] == 0).all()
    np.testing.assert_allclose(last["mean_a"], 1 - (1 - lam) ** 2, rtol=1e-12)


def test_eq3_committed_rows_are_token_embeddings():
    w = _tiny(boost_lo=12.0, boost_hi=14.0)
    W = run.weights(w)
    res = run.step(w, W=W, record_hidden=True)[0]
    n_commit = 0
    for rec in res["records"]:
        for i in np.nonzero(res["commit_loop"] != 0)[0]:
            if 0 < res["commit_loop"][i] <= rec["loop"]:
                assert np.array_equal(rec["h"][i], np.asarray(W["embed"][res["tokens"][i]], dtype=np.float64))
                n_commit += 1
        unres = np.nonzero(res["commit_loop"] == 0)[0]
        assert np.array_equal(rec["h"][unres], rec["h_tilde"][unres])
    assert n_commit > 0


def test_committed_tokens_are_planted_tokens_when_boost_dominates():
    w = _tiny(boost_lo=20.0, boost_hi=25.0, tau_ent=0.3)
    res = run.step(w)[0]
    tok, _ = synth.boosts(w)
    easy = tok[0] >= 0
    assert (res["commit_loop"][easy] == 1).all()
    assert np.array_equal(res["tokens"][easy], tok[0][easy])
    assert (res["commit_loop"][~easy] <= 0).all()


def test_thresholds_are_monotone():
    """Raising tau commits more rows at loop 1; raising q never runs fewer loops."""
    base = _tiny(boost_lo=8.0, boost_hi=14.0)
    W = run.weights(base)
    first = [int((run.step(replace(base, tau_ent=t), W=W)[0]["commit_loop"] == 1).sum())
             for t in (0.05, 0.3, 1.0, 3.0)]
    assert first == sorted(first) and first[-1] > first[0]
    loops = [run.step(replace(base, tau_ent=0.05, tau_halt=q), W=W)[0]["loops"] for q in (0.1, 0.5, 0.7, 0.95)]
    assert loops == sorted(loops) and loops[-1] > loops[0]


def test_layer_calls_without_prelude_and_coda():
    """The pages' 1.7B split (no Prelude, no Coda, Core = all 28 layers): K loops make 28 K layer
    calls, and the cache holds 28 K depth sets."""
    dims = replace(synth.QWEN3_8B_DIMS, vocab=64, d_model=16, n_q_heads=2, n_kv_heads=1, head_dim=8, ffn=16,
                   n_pre=0, n_core=28, n_coda=0)
    w = replace(_tiny(), dims=dims, prefix=3, block=4, k_max=4, tau_ent=-1.0, tau_halt=2.0)
    calls = []
    res = run.step(w, counter=calls)
    assert res[0]["loops"] == 4 and len(calls) == 4 * 28
    assert dims.kv_slots(4) == 112 and len(run.cache_for(w, run.weights(w), 0)) == 112


def test_first_loop_halt_mean_near_page_value():
    g = _golden("page_constants.json")["mean_first_pass_halt"]["value"]
    w = _tiny()
    lam = run.step(w)[0]["records"][0]["lam"]
    assert abs(float(np.nanmean(lam)) - g) < 0.1


def test_readout_group_reduces_to_step_rule():
    rng = np.random.default_rng(8)
    V, d = 50, 6
    Wl = rng.standard_normal((V, d))
    E = rng.standard_normal((V, d))
    r = rng.standard_normal((5, d))
    wg = rng.standard_normal(d)
    out = orc.readout_commit_group(r, Wl, E, wg, 0.1, tau_ent=1e9, tau_halt=0.5)
    assert (out["commit_loop"] == 1).all()
    np.testing.assert_array_equal(out["embed_rows"], E[out["tok"]])
    out = orc.readout_commit_group(r, Wl, E, wg, 0.1, tau_ent=-1.0, tau_halt=0.5)
    assert out["forced"] == int(np.argmin(out["H"])) and (out["commit_loop"] != 0).sum() == 1


def test_readout_group_halt_state():
    """The readout group's halting state after its one loop (summary page, Algorithm 1 (4)): the
    ExitGate logit of row i is set to logit(p_i) (w_g a unit vector, the row's first entry
    ln(p/(1-p)), b_g 0), so lambda_i = p_i exactly; from a = 0, a_i = lambda_i; mean_a is the mean
    of a over the rows the entropy commits left unresolved only, i.e. of the p_i of the rows that
    did not commit."""
    rng = np.random.default_rng(21)
    V, d = 40, 6
    Wl = rng.standard_normal((V, d))
    E = rng.standard_normal((V, d))
    p = np.array([0.2, 0.4, 0.6, 0.8, 0.9])
    r = rng.standard_normal((5, d))
    r[:, 0] = np.log(p / (1 - p))
    wg = np.zeros(d)
    wg[0] = 1.0
    H = orc.readout_commit_group(r, Wl, E, wg, 0.0, tau_ent=-1.0, tau_halt=0.5)["H"]
    order = np.argsort(H)
    tau = 0.5 * (H[order[1]] + H[order[2]])     # exactly the two rows of lowest entropy commit
    out = orc.readout_commit_group(r, Wl, E, wg, 0.0, tau_ent=tau, tau_halt=0.5)
    np.testing.assert_allclose(out["lam"], p, rtol=1e-12)
    np.testing.assert_allclose(out["a"], p, rtol=1e-12)
    left = np.setdiff1d(np.arange(5), order[:2])
    assert sorted(np.nonzero(out["commit_loop"] == 1)[0]) == sorted(order[:2]) and out["forced"] == -1
    np.testing.assert_allclose(out["mean_a"], p[left].mean(), rtol=1e-12)
    # nothing commits by entropy: the stop test (4) precedes forced progress (5), so every row is
    # still in the mean
    out = orc.readout_commit_group(r, Wl, E, wg, 0.0, tau_ent=-1.0, tau_halt=0.5)
    assert out["forced"] == order[0]
    np.testing.assert_allclose(out["mean_a"], p.mean(), rtol=1e-12)
    # every row commits: no unresolved row, no mean
    assert np.isnan(orc.readout_commit_group(r, Wl, E, wg, 0.0, tau_ent=1e9, tau_halt=0.5)["mean_a"])


def test_bf16_rounding_matches_library_conversion():
    import torch
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(10000) * 10.0 ** rng.integers(-6, 6, size=10000),
                        [1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]])
    ref = torch.tensor(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    got = orc.round_bf16(x)
    assert np.array_equal(got, ref)
    assert got[-5] == 1.0 and got[-4] == 1.0 and got[-3] == 1.0 + 2 ** -6   # ties to even


def test_rounding_points_mode_stays_close_to_exact():
    """The bf16 rounding-point variant of the step differs from the exact step by bf16 noise only."""
    w = _tiny(boost_lo=12.0, boost_hi=14.0)
    W = run.weights(w)
    a = run.step(w, W=W, record_hidden=True)[0]
    b = run.step(w, W=W, record_hidden=True, prec="bf16")[0]
    ra, rb = a["records"][0], b["records"][0]
    rel = np.linalg.norm(ra["h_tilde"] - rb["h_tilde"], axis=1) / np.linalg.norm(ra["h_tilde"], axis=1)
    assert 0 < rel.max() < 2e-2
    assert np.array_equal(a["commit_loop"], b["commit_loop"])


# --------------------------------------------------------------------------- sampling commit
def test_oracle_philox_known_answers():
    """The oracle's own Philox4x32-10 (independent of the input generator's) against the published
    known-answer vectors."""
    for v in _golden("philox4x32_10_kat.json")["vectors"]:
        c = [np.array([int(x, 16)]) for x in v["ctr"]]
        k = [int(x, 16) for x in v["key"]]
        out = orc.philox4x32_10(*c, *k)
        assert [int(x[0]) for x in out] == [int(x, 16) for x in v["out"]]


def test_gumbel_noise_range_and_counter_layout():
    """u = (floor(x / 2^9) + 1/2) / 2^23 lies in [2^-24, 1 - 2^-24], so g = -ln(-ln u) lies in
    [-ln(-ln 2^-24), -ln(-ln(1 - 2^-24))]; the noise of vocabulary id v is word v mod 4 of the
    block at counter v div 4, so a prefix of the vocabulary draws the same numbers."""
    g = orc.gumbel_noise(0x1234567890ABCDEF, 3, 2, 5, 1, 50001)
    lo = -math.log(-math.log(2.0 ** -24))
    hi = -math.log(-math.log1p(-2.0 ** -24))
    assert g.min() >= lo - 1e-12 and g.max() <= hi + 1e-12
    np.testing.assert_array_equal(orc.gumbel_noise(0x1234567890ABCDEF, 3, 2, 5, 1, 13), g[:13])
    # scalar definition through the input generator's separately written Philox, at ids that
    # cover every word of a block
    seed = 0x1234567890ABCDEF
    for v in (0, 1, 2, 3, 4, 7, 4097, 50000):
        x = int(synth.philox4x32_10([v // 4, 64 * 2 + 5, 1, 3], [seed & 0xFFFFFFFF, seed >> 32])[v % 4])
        u = ((x >> 9) + 0.5) / 2.0 ** 23
        assert g[v] == pytest.approx(-math.log(-math.log(u)), rel=1e-13, abs=1e-13)
    # standard Gumbel moments: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    assert abs(g.mean() - 0.5772156649) < 4 * math.sqrt(math.pi ** 2 / 6 / g.size)
    assert abs(g.var() - math.pi ** 2 / 6) < 0.05
    # every counter word matters: another row, loop, step or seed gives other noise
    for other in (orc.gumbel_noise(0x1234567890ABCDEF, 3, 2, 6, 1, 64), orc.gumbel_noise(0x1234567890ABCDEF, 3, 3, 5, 1, 64),
                  orc.gumbel_noise(0x1234567890ABCDEF, 3, 2, 5, 2, 64), orc.gumbel_noise(0x1234567890ABCDEF, 4, 2, 5, 1, 64),
                  orc.gumbel_noise(0x1234567890ABCDEE, 3, 2, 5, 1, 64), orc.gumbel_noise(0x0234567890ABCDEF, 3, 2, 5, 1, 64)):
        assert not np.array_equal(other, g[:64])


def test_gumbel_max_draws_follow_the_softmax():
    """argmax(z + g) over independent noise draws token v with probability softmax(z)_v: the
    empirical frequencies of 60000 draws sit within 4.5 standard errors of the softmax."""
    z = np.array([0.0, 1.0, 2.5, -1.0, 0.5, 2.0, -3.0])
    p = np.exp(z - z.max())
    p /= p.sum()
    n_i, n_s = 64, 6
    counts = np.zeros(z.size)
    n = 0
    for step in range(160):
        for b in range(1):
            for s in range(1, n_s + 1):
                G = np.stack([orc.gumbel_noise(99, step, b, i, s, z.size) for i in range(n_i)])
                tok, _ = orc.gumbel_sample(np.broadcast_to(z, G.shape), G)
                counts += np.bincount(tok, minlength=z.size)
                n += n_i
    f = counts / n
    se = np.sqrt(p * (1 - p) / n)
    assert (np.abs(f - p) < 4.5 * se).all(), (f, p)


def test_gumbel_sample_limits():
    """A logit 20 above every other always wins (the noise spans less than 20); equal logits draw
    every id; equal z + g goes to the lowest id."""
    V = 300
    z = np.zeros((40, V))
    z[:, 123] = 20.0
    G = np.stack([orc.gumbel_noise(5, 0, 0, i, 1, V) for i in range(40)])
    tok, gap = orc.gumbel_sample(z, G)
    assert (tok == 123).all() and (gap > 0).all()
    tok, _ = orc.gumbel_sample(np.zeros((40, V)), G)
    assert len(set(tok.tolist())) > 30
    t2, gap2 = orc.gumbel_sample(np.array([[1.0, 0.5, 1.0]]), np.array([[0.0, 0.5, 0.0]]))
    assert t2[0] == 0 and gap2[0] == 0


def test_sampled_step_equals_greedy_when_the_boost_dominates():
    """With planted boosts far above the noise span, every draw is the argmax, so the sampled step
    takes the greedy step's decisions exactly; with ordinary boosts it draws other tokens."""
    w = _tiny(boost_lo=30.0, boost_hi=34.0, tau_ent=0.3, batch=2)
    W = run.weights(w)
    g = run.step(w, W=W)
    s = run.step(w, W=W, sample=dict(seed=7, step=0))
    for a, b in zip(g, s):
        assert np.array_equal(a["tokens"], b["tokens"]) and np.array_equal(a["commit_loop"], b["commit_loop"])
        for ra, rb in zip(a["records"], b["records"]):
            rows = ra["rows"]
            assert np.array_equal(rb["stok"][rows][ra["H"][rows] < 1e-3], ra["tok"][rows][ra["H"][rows] < 1e-3])
    # near-uniform readout: draws differ from the argmax, commits take the draws
    w2 = _tiny(tau_ent=100.0)
    r2 = run.step(w2, sample=dict(seed=11, step=1))[0]
    rec = r2["records"][0]
    rows = rec["rows"]
    assert (r2["commit_loop"][rows] == 1).all()
    assert np.array_equal(r2["tokens"][rows], rec["stok"][rows])
    assert (rec["stok"][rows] != rec["tok"][rows]).sum() > rows.size // 2


def test_sampled_forced_commit_takes_the_draw():
    w = _tiny(tau_ent=-1.0, tau_halt=1.5)
    res = run.step(w, sample=dict(seed=3, step=2))[0]
    last = res["records"][-1]
    i = res["forced"]
    assert i == int(np.argmin(last["H"])) and res["tokens"][i] == last["stok"][i]
    assert res["commit_loop"][i] == -w.k_max


# --------------------------------------------------------------------------- outer loop and cache growth
def test_extend_equals_prefill_of_the_longer_prefix():
    """By causality, appending positions to a full-depth cache gives the prefill of the longer
    prefix, whether appended at once, in pieces, or onto an empty cache."""
    w = _tiny()
    W = _rand_weights(w)
    ids = np.random.default_rng(5).integers(0, w.dims.vocab, size=20)
    kw = dict(dims=w.dims, k_max=w.k_max, eps=w.rms_eps, theta=w.rope_theta)
    full = orc.prefill_sequence(ids, W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
    part = orc.prefill_sequence(ids[:12], W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
    one, av1 = orc.extend_sequence(part, None, ids[12:], W, **kw)
    two, _ = orc.extend_sequence(part, None, ids[12:15], W, **kw)
    two, av2 = orc.extend_sequence(two, None, ids[15:], W, **kw)
    empty, _ = orc.extend_sequence({}, None, ids[:8], W, **kw)
    ref8 = orc.prefill_sequence(ids[:8], W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
    assert sorted(one) == sorted(full) and (av1 == w.k_max).all() and av2.shape == (20,)
    for slot in full:
        for a, b, c in zip(one[slot], two[slot], full[slot]):
            np.testing.assert_allclose(a, c, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(b, c, rtol=1e-11, atol=1e-12)
        for a, c in zip(empty[slot], ref8[slot]):
            np.testing.assert_allclose(a, c, rtol=1e-11, atol=1e-12)


def test_extend_reads_cached_positions_at_their_available_depth():
    """Cached positions with available depth 1 are read at depth 1 by every Core pass of the
    appended positions: the same as a cache whose deeper Core slots hold the depth-1 values."""
    w = _tiny()
    W = _rand_weights(w, seed=2)
    D = w.dims
    ids = np.random.default_rng(6).integers(0, D.vocab, size=14)
    kw = dict(dims=D, k_max=w.k_max, eps=w.rms_eps, theta=w.rope_theta)
    cache = orc.prefill_sequence(ids[:10], W, D, w.k_max, w.rms_eps, w.rope_theta)
    flat = dict(cache)
    for c in range(D.n_core):
        for dpt in range(2, w.k_max + 1):
            flat[orc.kv_slot(D, w.k_max, D.n_pre + c, dpt)] = cache[orc.kv_slot(D, w.k_max, D.n_pre + c, 1)]
    a, _ = orc.extend_sequence(cache, np.ones(10, dtype=int), ids[10:], W, **kw)
    b, _ = orc.extend_sequence(flat, None, ids[10:], W, **kw)
    c, _ = orc.extend_sequence(cache, None, ids[10:], W, **kw)
    deep = orc.kv_slot(D, w.k_max, D.n_pre, w.k_max)
    for slot in a:
        np.testing.assert_allclose(a[slot][0][:, 10:], b[slot][0][:, 10:], rtol=1e-11, atol=1e-12)
    assert not np.allclose(a[deep][0][:, 10:], c[deep][0][:, 10:])


def test_outer_loop_resolves_every_mask():
    w = _tiny(boost_lo=8.0, boost_hi=14.0, batch=2)
    bids = synth.block_ids(w)
    bids[1, [2, 3, 9]] = [11, 12, 13]
    res = run.denoise_block(w, block_ids=bids)
    for r in res:
        b = r["seq"]
        masked = bids[b] == w.mask_id
        assert (r["tokens"] != w.mask_id).all() and np.array_equal(r["tokens"][~masked], bids[b][~masked])
        assert (r["commit_step"][masked] >= 1).all() and (r["commit_step"][~masked] == 0).all()
        assert 1 <= r["steps"] <= masked.sum()
        assert all(int((st["commit_loop"] != 0).sum()) >= 1 for st in r["results"])
        assert r["steps"] < masked.sum()          # entropy commits: several tokens in some step
    # the first step is the plain step
    first = run.step(w, block_ids=bids)
    for r, f in zip(res, first):
        assert np.array_equal(r["results"][0]["tokens"], f["tokens"])


def test_one_token_per_step_mode():
    """tau_ent < 0 commits nothing by entropy, so every step commits exactly its forced token: a
    block with n masks takes n steps, one position each."""
    w = _tiny(tau_ent=-1.0, tau_halt=0.5)
    r = run.denoise_block(w)[0]
    masked = synth.block_ids(w)[0] == w.mask_id
    n = int(masked.sum())
    assert r["steps"] == n
    assert sorted(r["commit_step"][masked].tolist()) == list(range(1, n + 1))
    assert (r["commit_loop"][masked] < 0).all()


def test_no_mask_no_loop_and_sampled_steps_advance_the_counter():
    w = _tiny(tau_ent=4.0)
    full = synth.block_ids(w)
    full[:] = 5
    r = run.step(w, block_ids=full)[0]
    assert r["loops"] == 0 and r["records"] == [] and (r["commit_loop"] == 0).all()
    assert run.denoise_block(w, block_ids=full)[0]["steps"] == 0
    blk = run.denoise_block(w, sample=dict(seed=9, step0=5))[0]
    assert blk["steps"] >= 2
    ids1 = np.asarray(blk["results"][0]["tokens"])
    again = run.step(w, block_ids=ids1[None, :], sample=dict(seed=9, step=6))[0]
    assert np.array_equal(again["tokens"], blk["results"][1]["tokens"])


def test_depth_on_demand_prefill_then_deepen_equals_full_prefill():
    """Building depth 1 first and deepening later gives the full-depth cache; before deepening,
    a step reads the deeper Core planes at depth 1."""
    w = _tiny()
    W = _rand_weights(w, seed=3)
    D = w.dims
    ids = np.random.default_rng(7).integers(0, D.vocab, size=18)
    args = (W, D, w.k_max, w.rms_eps, w.rope_theta)
    full = orc.prefill_sequence(ids, *args)
    c1, s1 = orc.prefill_sequence(ids, *args, depth=1, state=True)
    assert sorted(c1) == sorted(set(range(D.n_pre)) | {orc.kv_slot(D, w.k_max, D.n_pre + c, 1) for c in range(D.n_core)}
                                | {orc.kv_slot(D, w.k_max, D.n_pre + D.n_core + c) for c in range(D.n_coda)})
    c2, s2 = orc.deepen_sequence(c1, s1, *args, depth_from=1, depth_to=2)
    c4, _ = orc.deepen_sequence(c2, s2, *args, depth_from=2, depth_to=w.k_max)
    assert sorted(c4) == sorted(full)
    for slot in full:
        for a, b in zip(c4[slot], full[slot]):
            np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    c2d = orc.prefill_sequence(ids, *args, depth=2)
    for slot in c2d:
        for a, b in zip(c2[slot], c2d[slot]):
            np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    # the Coda set of a shallow build comes from the shallow output
    coda = orc.kv_slot(D, w.k_max, D.n_pre + D.n_core)
    assert not np.allclose(c1[coda][0], full[coda][0])


# --------------------------------------------------------------------------- fp8 K/V storage
def _e4m3_table():
    """Every finite OCP FP8 E4M3 value from the format definition: sign, 4 exponent bits (bias 7),
    3 fraction bits; exponent field 0 is subnormal (f/8 * 2^-6); code S.1111.111 is NaN."""
    vals = []
    for code in range(256):
        s, e, f = code >> 7, (code >> 3) & 15, code & 7
        if e == 15 and f == 7:
            continue
        v = (f / 8.0) * 2.0 ** -6 if e == 0 else (1 + f / 8.0) * 2.0 ** (e - 7)
        vals.append(-v if s else v)
    return np.array(sorted(set(vals)))


def test_fp8_rounding_fixed_points_and_range():
    t = _e4m3_table()
    assert t.max() == 448.0 and t.min() == -448.0 and np.min(t[t > 0]) == 2.0 ** -9 and t.size == 253
    np.testing.assert_array_equal(orc.round_fp8_e4m3(t), t)
    x = np.random.default_rng(11).uniform(-500, 500, 20000) * np.random.default_rng(12).choice(
        [1.0, 1e-1, 1e-2, 1e-3], 20000)
    r = orc.round_fp8_e4m3(x)
    assert np.isin(r, t).all()
    # nearest representable value (ties resolved below)
    idx = np.searchsorted(t, x)
    lo, hi = t[np.clip(idx - 1, 0, t.size - 1)], t[np.clip(idx, 0, t.size - 1)]
    best = np.where(np.abs(x - lo) <= np.abs(x - hi), lo, hi)
    inside = np.abs(x) <= 448.0
    tie = np.abs(np.abs(x - lo) - np.abs(x - hi)) < 1e-12
    assert (r[inside & ~tie] == best[inside & ~tie]).all()
    assert (orc.round_fp8_e4m3(np.array([460.0, 1000.0, -1e6])) == [448.0, 448.0, -448.0]).all()


def test_fp8_rounding_matches_library_conversion():
    """Against torch's float32 -> float8_e4m3fn conversion (round to nearest even) inside the finite
    range, including every midpoint between neighbouring values (ties to the even code)."""
    t = _e4m3_table()
    mids = (t[1:] + t[:-1]) / 2
    x = np.concatenate([mids, np.random.default_rng(13).normal(0, 3, 50000), t])
    x = x[np.abs(x) <= 448.0].astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.round_fp8_e4m3(x), lib)


def test_fp8_cache_holds_e4m3_values_and_changes_little():
    w = _tiny(dtype="bf16")
    W = run.weights(w)
    ids = synth.prefix_ids(w)[0]
    c8 = orc.prefill_sequence(ids, W, w.dims, w.k_max, w.rms_eps, w.rope_theta, kv="fp8")
    c = orc.prefill_sequence(ids, W, w.dims, w.k_max, w.rms_eps, w.rope_theta)
    for slot in c:
        for a8, a in zip(c8[slot], c[slot]):
            np.testing.assert_array_equal(orc.round_fp8_e4m3(a8), a8)
            rel = np.linalg.norm(a8 - a) / np.linalg.norm(a)
            assert 1e-4 < rel < 0.08
    r8 = run.step(replace(w, kv_dtype="fp8"), W=W)[0]
    r = run.step(w, W=W)[0]
    h8 = r8["records"][0]["H"][r8["records"][0]["rows"]]
    h = r["records"][0]["H"][r["records"][0]["rows"]]
    assert 0 < np.abs(h8 - h).max() < 0.1


def test_batch_depth_on_demand_policy_reduces_to_the_plain_outer_loop():
    """Built to full depth, the on-demand policy never deepens and equals the per-sequence outer loop;
    built to depth 1 it deepens to the first step's loop count."""
    w = _tiny(batch=2, boost_lo=8.0, boost_hi=14.0, tau_ent=0.8, tau_halt=0.6)
    W = run.weights(w)
    full = run.denoise_block_on_demand(w, w.k_max, W=W)
    plain = run.denoise_block(w, W=W)
    assert full["depth_after_step"] == [w.k_max] * full["steps"]
    for r in plain:
        b = r["seq"]
        assert np.array_equal(full["tokens"][b], r["tokens"]) and np.array_equal(full["commit_step"][b], r["commit_step"])
    od = run.denoise_block_on_demand(w, 1, W=W)
    first = max(res["loops"] for (t, _, res) in od["results"] if t == 1)
    assert od["depth_after_step"][0] == max(1, first) and od["built_depth"] == max(od["depth_after_step"])


# --------------------------------------------------------------------------- depth eviction
def test_evict_depths_buffer_counts_match_page():
    """Keeping one Core depth leaves the autoregressive model's buffer count, keeping all K the
    page's 84; the kept sets are the Prelude, the Coda and Core depths 1..D; depths are clipped."""
    g = _golden("page_constants.json")
    d8 = synth.QWEN3_8B_DIMS
    K = g["k_loops"]["value"]
    full = {s: (s, s) for s in range(d8.kv_slots(K))}
    for D, n in ((1, g["kv_buffers_8b_k4"]["autoregressive_value"]), (K, g["kv_buffers_8b_k4"]["value"]),
                 (2, d8.n_layers + d8.n_core)):
        kept, av = orc.evict_depths(full, None, d8, K, D, 5)
        assert len(kept) == n == d8.kv_slots(D)
        assert set(kept) == {orc.kv_slot(d8, K, l, dp) for l in range(d8.n_layers)
                             for dp in range(1, (D if d8.n_pre <= l < d8.n_pre + d8.n_core else 1) + 1)}
        assert all(kept[s] == full[s] for s in kept) and (av == D).all()
    _, av = orc.evict_depths({}, np.array([1, 2, 3, 4, 4]), d8, K, 2, 5)
    assert av.tolist() == [1, 2, 2, 2, 2]


def test_step_on_evicted_cache_reads_the_deepest_kept_depth():
    """With one depth kept, a step equals the step on a full cache whose every Core plane holds
    the depth-1 sets (the fallback written out by hand); it differs from the full-depth step once
    a loop runs past depth 1."""
    w = _tiny(tau_ent=0.3, tau_halt=0.9)
    W = run.weights(w)
    D = w.dims
    cache = run.cache_for(w, W, 0)
    flat = dict(cache)
    for c in range(D.n_core):
        for dpt in range(2, w.k_max + 1):
            flat[orc.kv_slot(D, w.k_max, D.n_pre + c, dpt)] = cache[orc.kv_slot(D, w.k_max, D.n_pre + c, 1)]
    w1 = replace(w, cache_depths=1)
    ev = run.cache_for(w1, W, 0)
    assert len(ev) == D.kv_slots(1)
    r_ev = run.step(w1, W=W, seqs=[0], record_hidden=True)[0]
    r_flat = run.step(w, W=W, seqs=[0], caches={0: flat}, record_hidden=True)[0]
    r_full = run.step(w, W=W, seqs=[0], record_hidden=True)[0]
    assert r_ev["loops"] >= 2 and r_ev["loops"] == r_flat["loops"]
    for a, b in zip(r_ev["records"], r_flat["records"]):
        np.testing.assert_allclose(a["h_tilde"], b["h_tilde"], rtol=1e-12, atol=1e-13)
    assert not np.allclose(r_ev["records"][1]["h_tilde"], r_full["records"][1]["h_tilde"])
    np.testing.assert_allclose(r_ev["records"][0]["h_tilde"], r_full["records"][0]["h_tilde"], rtol=1e-12,
                               atol=1e-13)


def test_extend_on_evicted_cache():
    """Appending to a cache that keeps D depths: the new positions' Prelude and Core depth 1..D sets
    equal those of the full-cache extension (those passes read cached positions at depth <= D
    either way) while the Coda set differs; with every cached position at depth <= D, extending
    then evicting equals evicting then extending."""
    w = _tiny()
    W = _rand_weights(w, seed=4)
    D = w.dims
    ids = np.random.default_rng(8).integers(0, D.vocab, size=16)
    kw = dict(dims=D, k_max=w.k_max, eps=w.rms_eps, theta=w.rope_theta)
    cache = orc.prefill_sequence(ids[:11], W, D, w.k_max, w.rms_eps, w.rope_theta)
    ev, av = orc.evict_depths(cache, None, D, w.k_max, 2, 11)
    a, av_a = orc.extend_sequence(ev, av, ids[11:], W, keep=2, **kw)
    b, _ = orc.extend_sequence(cache, None, ids[11:], W, **kw)
    assert sorted(a) == sorted(ev) and av_a.tolist() == [2] * 16
    coda = orc.kv_slot(D, w.k_max, D.n_pre + D.n_core)
    for slot in a:
        same = np.allclose(a[slot][0][:, 11:], b[slot][0][:, 11:], rtol=1e-11, atol=1e-12)
        assert same == (slot < coda), slot
    # every cached position at depth <= 2: eviction commutes with the extension
    shallow = np.array([1, 2] * 5 + [2])
    ev2, av2 = orc.evict_depths(cache, shallow, D, w.k_max, 2, 11)
    c, _ = orc.extend_sequence(ev2, av2, ids[11:], W, keep=2, **kw)
    full2, avf = orc.extend_sequence(cache, shallow, ids[11:], W, **kw)
    d_, _ = orc.evict_depths(full2, avf, D, w.k_max, 2, 16)
    assert sorted(c) == sorted(d_)
    for slot in c:
        for x, y in zip(c[slot], d_[slot]):
            np.testing.assert_allclose(x, y, rtol=1e-11, atol=1e-12)


def test_near_decision_flags_fire_exactly_inside_their_thresholds():
    """The flags that exempt an outer-loop sequence from the exact free-run comparison: an entropy
    within the threshold of tau_ent, a committed token whose top-2 gap is within it, a halting mean
    within it of tau_halt, a forced commit whose entropy gap or token gap is within it -- and
    nothing else."""
    w = _tiny(tau_ent=0.5, tau_halt=0.6)
    nan = float("nan")

    def rec(H, gap, committed, mean_a, n_u=3):
        return dict(loop=1, rows=np.arange(4), H=np.asarray(H, float), gap=np.asarray(gap, float),
                    committed=np.asarray(committed, int), mean_a=mean_a, n_unresolved=n_u)

    def res(r, forced=-1, forced_gap=nan):
        return dict(records=[r], forced=forced, forced_gap=forced_gap)

    far = rec([3.0, 4.0, 0.2, 5.0], [1.0, 1.0, 0.5, 1.0], [2], 0.3)
    assert run.near_decisions(w, res(far)) == []
    for H in (0.495, 0.505, 0.5):
        assert any("entropy" in f for f in run.near_decisions(w, res(rec([3.0, 4.0, H, 5.0], [1, 1, 1, 1], [], 0.3))))
    assert run.near_decisions(w, res(rec([3.0, 4.0, 0.48, 5.0], [1, 1, 1, 1], [2], 0.3))) == []
    assert run.near_decisions(w, res(rec([3.0, 4.0, 0.2, 5.0], [1, 1, 0.005, 1], [2], 0.3))) == [
        "token gap loop 1 row 2"]
    assert run.near_decisions(w, res(rec([3.0, 4.0, 0.2, 5.0], [1, 0.005, 1, 1], [2], 0.3))) == []  # row 1 not committed
    assert run.near_decisions(w, res(rec([3.0, 4.0, 0.2, 5.0], [1, 1, 1, 1], [2], 0.605))) == ["halt loop 1"]
    assert run.near_decisions(w, res(rec([3.0, 4.0, 0.2, 5.0], [1, 1, 1, 1], [2], 0.605, n_u=0))) == []
    assert run.near_decisions(w, res(rec([3.0, 4.0, 2.2, 5.0], [1, 1, 1, 1], [], 0.3), forced=2, forced_gap=0.004)) == [
        "forced entropy gap"]
    assert run.near_decisions(w, res(rec([3.0, 4.0, 2.2, 5.0], [1, 1, 0.001, 1], [], 0.3), forced=2, forced_gap=0.8)) \
        == ["forced token gap"]
