"""C-ABI checks that need no GPU: the library loads, exports every declared entry point, and
rejects bad arguments before any device work."""
import ctypes
import os
import re
from dataclasses import replace

import pytest

from adaptive_looped_denoising_amd import binding as B
from adaptive_looped_denoising_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for h in ("alodlm.h", "alodlm_synth.h", "alodlm_diag.h"):
        txt = open(os.path.join(ROOT, "include", h)).read()
        names |= set(re.findall(r"\b(alodlm_[a-z_0-9]+)\s*\(", txt))
    return names


def _cfg(w=None, **over):
    w = w or synth.workload("qwen3_8b")
    D = w.dims
    c = B.Config(vocab=D.vocab, d_model=D.d_model, n_q_heads=D.n_q_heads, n_kv_heads=D.n_kv_heads,
                 head_dim=D.head_dim, ffn=D.ffn, n_pre=D.n_pre, n_core=D.n_core, n_coda=D.n_coda, k_max=w.k_max,
                 max_batch=w.batch, max_prefix=w.prefix, max_block=w.block, max_prefill_rows=0, mask_id=w.mask_id,
                 dtype=B.DTYPE_BF16 if w.dtype == "bf16" else B.DTYPE_FP32, rms_eps=w.rms_eps,
                 rope_theta=w.rope_theta)
    for k, v in over.items():
        setattr(c, k, v)
    return c


def test_library_loads_and_exports_every_declared_symbol():
    lib = B.load()
    declared = _declared()
    assert {"alodlm_create", "alodlm_prefill_kv", "alodlm_denoise_step", "alodlm_destroy"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(B.EXPORTS) == declared


def test_kv_slot_counts():
    assert B.kv_slots(_cfg()) == 84                    # 8B split at K = 4
    assert B.kv_slots(_cfg(synth.workload("qwen3_8b_long"))) == 116
    assert B.kv_slots(_cfg(synth.workload("tiny"))) == 1 + 2 * 4 + 1


def test_workspace_size_covers_the_cache():
    c = _cfg()
    n = B.workspace_bytes(c)
    kv = 2 * 84 * 8 * 8 * 1024 * 128 * 2
    assert kv < n < kv + 3 * 2 ** 30
    c4 = _cfg(synth.workload("qwen3_8b_long"), max_prefill_rows=8192)
    assert B.workspace_bytes(c4) > 2 * 116 * 32 * 8 * 8192 * 128 * 2


@pytest.mark.parametrize("field,value", [
    ("dtype", 7), ("vocab", 1), ("d_model", 100), ("ffn", 0), ("head_dim", 48), ("n_q_heads", 3),
    ("n_kv_heads", 0), ("n_core", 0), ("n_pre", -1), ("k_max", 0), ("k_max", 17), ("max_batch", 0),
    ("max_batch", 2000), ("max_block", 65), ("max_block", 0), ("max_prefix", -2), ("max_prefill_rows", 5),
    ("mask_id", 151936), ("rms_eps", float("nan")), ("rope_theta", 0.0), ("depth_on_demand", 2),
    ("kv_dtype", 1), ("kv_dtype", 3)])
def test_bad_configs_are_rejected(field, value):
    with pytest.raises(B.AlodlmError) as e:
        B.workspace_bytes(_cfg(**{field: value}))
    assert e.value.code == B.EINVAL
    assert "invalid config" in str(e.value)


def test_fp8_kv_config_rules_and_workspace():
    """fp8 keys and values need the bf16 dtype and head_dim 64 or 128, and halve the cache bytes;
    depth-on-demand adds the prefix state [max_batch][max_prefix][d] fp32."""
    for w in (synth.workload("tiny"), replace(synth.workload("tiny"), dtype="bf16")):   # hd 32 / fp32
        with pytest.raises(B.AlodlmError) as e:
            B.workspace_bytes(_cfg(w, kv_dtype=B.KV_FP8))
        assert e.value.code == B.EINVAL
    base = B.workspace_bytes(_cfg())
    f8 = B.workspace_bytes(_cfg(kv_dtype=B.KV_FP8))
    kv = 2 * 84 * 8 * 8 * 1024 * 128 * 2
    assert abs((base - f8) - kv / 2) < 64 * 2 ** 20      # the cache (and own-block K/V) at one byte
    dod = B.workspace_bytes(_cfg(depth_on_demand=1))
    assert abs((dod - base) - 8 * 1024 * 4096 * 4) < 2 ** 20


def test_depth_eviction_config_rules_and_workspace():
    """cache_depths D in 0..k_max keeps Core depths 1..D: n_pre + n_core * D + n_coda slots plus one
    scratch plane for the deeper passes; with depth-on-demand only 0 or k_max."""
    for bad in (-1, 5):
        with pytest.raises(B.AlodlmError) as e:
            B.workspace_bytes(_cfg(cache_depths=bad))
        assert e.value.code == B.EINVAL
    for D in (1, 2, 3):
        with pytest.raises(B.AlodlmError) as e:
            B.workspace_bytes(_cfg(cache_depths=D, depth_on_demand=1))
        assert e.value.code == B.EINVAL
    assert B.workspace_bytes(_cfg(cache_depths=4, depth_on_demand=1)) == B.workspace_bytes(_cfg(depth_on_demand=1))
    base = B.workspace_bytes(_cfg())
    assert B.kv_slots(_cfg()) == B.kv_slots(_cfg(cache_depths=4)) == 84 and B.workspace_bytes(_cfg(cache_depths=4)) == base
    plane = 2 * 8 * 8 * 1024 * 128 * 2          # K and V of one slot: B * Hkv * P * hd bf16
    for D in (1, 2, 3):
        assert B.kv_slots(_cfg(cache_depths=D)) == 36 + 16 * (D - 1)
        saved = base - B.workspace_bytes(_cfg(cache_depths=D))
        assert saved == (16 * (4 - D) - 1) * plane


def _weights(nl, ptr=0x1000):
    layers = (B.LayerWeights * nl)()
    for l in range(nl):
        for f, _ in B.LayerWeights._fields_:
            setattr(layers[l], f, ptr)
    return B.Weights(embed=ptr, lm_head=ptr, final_norm=ptr, exit_w=ptr, exit_b=0.1, layers=layers), layers


def test_create_validates_before_device_work():
    lib = B.load()
    c = _cfg(synth.workload("tiny"))
    w, keep = _weights(4)
    need = B.workspace_bytes(c)
    out = ctypes.c_void_p(0)
    # workspace too small
    rc = lib.alodlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(0x10000), need - 1, None,
                           ctypes.byref(out))
    assert rc == B.ENOMEM and out.value is None
    assert b"need" in lib.alodlm_last_error(None)
    # misaligned workspace
    rc = lib.alodlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(0x10010), need, None, ctypes.byref(out))
    assert rc == B.EINVAL
    # a null layer tensor
    keep[2].wo = None
    rc = lib.alodlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(0x10000), need, None, ctypes.byref(out))
    assert rc == B.EINVAL and b"layer 2" in lib.alodlm_last_error(None)
    # non-finite exit bias
    keep[2].wo = 0x1000
    w.exit_b = float("inf")
    rc = lib.alodlm_create(ctypes.byref(c), ctypes.byref(w), ctypes.c_void_p(0x10000), need, None, ctypes.byref(out))
    assert rc == B.EINVAL


def test_null_context_calls_fail_cleanly():
    lib = B.load()
    assert lib.alodlm_prefill_kv(None, 1, 1, None, None) == B.EINVAL
    assert lib.alodlm_denoise_step(None, None, None) == B.EINVAL
    assert lib.alodlm_readout_commit(None, None, 32, 32, 0.5, 0.5, *([None] * 10)) == B.EINVAL
    assert lib.alodlm_last_step_stats(None, None, None) == B.EINVAL
    assert lib.alodlm_extend_kv(None, 1, 1, None, None) == B.EINVAL
    assert lib.alodlm_denoise_block(None, None, None) == B.EINVAL
    assert lib.alodlm_prefill_kv_depth(None, 1, 1, None, 1) == B.EINVAL
    assert lib.alodlm_deepen_kv(None, 2) == B.EINVAL
    lib.alodlm_destroy(None)
    assert lib.alodlm_synth_fill(None, 0, 0, 10, 0, 0, 1.0, 0.0, None) == -1
    # diagnostics entry: bad shapes and null operands are rejected before any launch
    assert lib.alodlm_diag_readout_sample(0, 10, 64, None, None, None, 1, 1, 1, None, None, 0, 0, -1, None) == -1


def _fake_ctx(w, **over):
    """A context over fake device pointers: creation and argument checks touch no device."""
    lib = B.load()
    c = _cfg(w, **over)
    wts, keep = _weights(w.dims.n_layers)
    need = B.workspace_bytes(c)
    out = ctypes.c_void_p(0)
    rc = lib.alodlm_create(ctypes.byref(c), ctypes.byref(wts), ctypes.c_void_p(0x10000), need, None,
                           ctypes.byref(out))
    assert rc == B.OK and out.value
    return lib, out.value, (wts, keep)


def test_create_makes_no_device_call_and_calls_validate_first():
    """Creation is host only, so every entry point's argument checks run here without a device."""
    w = synth.workload("qwen3_8b")
    lib, ctx, keep = _fake_ctx(w)
    try:
        cx = ctypes.c_void_p(ctx)
        # a step or an append before any prefill
        args = B.StepArgs(batch=8, block_len=32, block_ids=0x1000, tau_ent=0.6, tau_halt=0.5, k_loops=4)
        out = B.StepOut(tokens=0x1000, commit_loop=0x1000, loops=0x1000)
        assert lib.alodlm_denoise_step(cx, ctypes.byref(args), ctypes.byref(out)) == B.ESTATE
        assert lib.alodlm_extend_kv(cx, 8, 32, ctypes.c_void_p(0x1000), None) == B.ESTATE
        assert lib.alodlm_deepen_kv(cx, 2) == B.EINVAL            # not a depth-on-demand config
        # prefill arguments out of range
        assert lib.alodlm_prefill_kv(cx, 9, 1024, ctypes.c_void_p(0x1000), None) == B.EINVAL
        assert lib.alodlm_prefill_kv(cx, 8, 1025, ctypes.c_void_p(0x1000), None) == B.EINVAL
        assert lib.alodlm_prefill_kv(cx, 8, 1024, None, None) == B.EINVAL
        assert lib.alodlm_prefill_kv_synthetic(cx, 8, 1024, 1, float("nan"), 1.0, None) == B.EINVAL
        assert lib.alodlm_prefill_kv_depth(cx, 8, 1024, ctypes.c_void_p(0x1000), 1) == B.EINVAL
    finally:
        lib.alodlm_destroy(ctypes.c_void_p(ctx))


@pytest.mark.parametrize("n_rows,group,why", [
    (32, 0, b"group"), (32, 65, b"group"), (96, 64, b"group"), (0, 32, b"n_rows"), (257, 1, b"n_rows"),
    (256, 16, b"max_batch"), (64, 1, b"max_batch"), (256, 31, b"group")])
def test_readout_commit_rejects_groups_beyond_the_sequence_state(n_rows, group, why):
    """The readout entry point's per-sequence state holds max_batch sequences: n_rows / group above
    that (here max_batch 8, 8 x 32 rows) is rejected before any device work."""
    w = synth.workload("qwen3_8b")
    lib, ctx, keep = _fake_ctx(w)
    try:
        cx = ctypes.c_void_p(ctx)
        p = ctypes.c_void_p(0x1000)
        rc = lib.alodlm_readout_commit(cx, p, n_rows, group, 0.6, 0.5, None, None, *([p] * 8))
        assert rc == B.EINVAL
        assert why in lib.alodlm_last_error(cx)
        # non-finite thresholds and a boost token array without values
        rc = lib.alodlm_readout_commit(cx, p, 256, 32, float("inf"), 0.5, None, None, *([p] * 8))
        assert rc == B.EINVAL
        rc = lib.alodlm_readout_commit(cx, p, 256, 32, 0.6, 0.5, p, None, *([p] * 8))
        assert rc == B.EINVAL
    finally:
        lib.alodlm_destroy(ctypes.c_void_p(ctx))


def test_static_readout_validates_and_bounds_its_scratch():
    """The allocation-free readout takes the same argument checks, and rejects a readout whose
    scratch would not fit the library's fixed array (checked before any device call)."""
    w = synth.workload("qwen3_8b")
    lib, ctx, keep = _fake_ctx(w)
    p = ctypes.c_void_p(0x1000)
    try:
        cx = ctypes.c_void_p(ctx)
        assert lib.alodlm_readout_commit_static(cx, p, 256, 16, 0.6, 0.5, None, None, *([p] * 8)) == B.EINVAL
        assert b"max_batch" in lib.alodlm_last_error(cx)
        assert lib.alodlm_readout_commit_static(cx, None, 256, 32, 0.6, 0.5, None, None, *([p] * 8)) == B.EINVAL
    finally:
        lib.alodlm_destroy(ctypes.c_void_p(ctx))
    # 2048 rows over a 4M-token vocabulary: 16 B x 2048 x 15625 tiles of statistics > 32 MiB
    big = replace(w, batch=64, dims=replace(w.dims, vocab=4_000_000))
    lib, ctx, keep = _fake_ctx(big, mask_id=4_000_000 - 1)
    try:
        cx = ctypes.c_void_p(ctx)
        assert lib.alodlm_readout_commit_static(cx, p, 2048, 32, 0.6, 0.5, None, None, *([p] * 8)) == B.EINVAL
        assert b"scratch" in lib.alodlm_last_error(cx)
    finally:
        lib.alodlm_destroy(ctypes.c_void_p(ctx))


@pytest.mark.parametrize("pad,ok", [(0, True), (64, True), (1024, True), (4, False), (-8, False), (1032, False)])
def test_weight_row_pad_range(pad, ok):
    """weight_row_pad: a multiple of 8 (16-byte aligned rows for the matrix-core loads) in 0..1024."""
    if ok:
        assert B.workspace_bytes(_cfg(weight_row_pad=pad)) > 0
    else:
        with pytest.raises(B.AlodlmError) as e:
            B.workspace_bytes(_cfg(weight_row_pad=pad))
        assert e.value.code == B.EINVAL


def test_swiglu_few_rows_tiles():
    """FFN gate/up at up to 64 rows: the eight-wave 64 x 128 tile when its N / 128 workgroups cover
    three quarters of the compute units (the 8B width), else the four-wave 64 x 64 tile (the 1.7B
    width); single pass (the SwiGLU epilogue needs no split-K reduction)."""
    for M in (1, 32, 48, 64):
        t, sp, name = B.gemm_choice(3, M, 2 * 6144, 2048, 8 * M * 2 * 6144)
        assert (t, sp) == (12, 1) and name.startswith("k_gemm_pipe<64, 64,"), (M, name)
        t, sp, name = B.gemm_choice(3, M, 2 * 12288, 4096, 8 * M * 2 * 12288)
        assert (t, sp) == (45, 1) and name.startswith("k_gemm_pipe<64, 128,"), (M, name)


def test_readout_column_ranges():
    """The LM-head readout's column split (host-side plan): a 256-row readout over the 8B vocabulary
    runs the 512 whole rounds of 256 x 256 tiles and the remaining 20864 columns on the
    eight-wave tile; fewer rows, several row tiles or a vocabulary filling its last round stay in
    one launch."""
    V, d = 151936, 4096
    t, _, name = B.gemm_choice(2, 256, V, d, 0)
    assert t == 64 and "(columns 0..131071)" in name and "(columns 131072..151935)" in name, name
    assert name.startswith("k_gemm_pipe<256, 256, 4, 2, 2, 2, false> (columns 0..131071)"), name
    assert name.count("k_gemm_") == 2
    for M, N in ((224, V), (129, V)):
        assert "(columns 0..131071)" in B.gemm_choice(2, M, N, d, 0)[2]
    for M, N in ((128, V), (300, V), (2048, V), (256, 256 * 512), (256, 256 * 512 + 256 * 200), (256, 4096)):
        assert "columns" not in B.gemm_choice(2, M, N, d, 0)[2], (M, N)
