"""ctypes binding of libalodlm.so (argument marshalling only; every step runs in the HIP library).

The names mirror the C ABI in include/alodlm.h.  Loading fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int8, c_int32, c_int64, c_size_t, c_uint32, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libalodlm.so")

OK, EINVAL, ESTATE, ENOMEM, EHIP = 0, -1, -2, -3, -4
DTYPE_BF16, DTYPE_FP32 = 0, 1
KV_SAME, KV_FP8 = 0, 2
STEP_TEACHER_FORCED, STEP_SAMPLE = 1, 2
# diagnostics GEMM epilogues (alodlm_diag.h)
DIAG_STORE, DIAG_RESID, DIAG_SOFTSTAT, DIAG_SWIGLU = 0, 1, 2, 3

EXPORTS = ("alodlm_workspace_bytes", "alodlm_kv_slots", "alodlm_create", "alodlm_prefill_kv",
           "alodlm_prefill_kv_synthetic", "alodlm_prefill_kv_depth", "alodlm_deepen_kv", "alodlm_extend_kv", "alodlm_denoise_step", "alodlm_denoise_block",
           "alodlm_readout_commit", "alodlm_readout_commit_static",
           "alodlm_last_step_stats", "alodlm_last_error", "alodlm_destroy", "alodlm_synth_fill",
           "alodlm_diag_gemm", "alodlm_diag_timing_enable", "alodlm_diag_timing_read", "alodlm_diag_read_kv", "alodlm_diag_buffer_offset",
           "alodlm_diag_readout_sample", "alodlm_diag_gemm_choice")
K_CLASSES = ("gemm_gate_up", "gemm_qkv", "gemm_o", "gemm_down", "attention", "lm_head", "norm_rope", "control")


class Config(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "vocab", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "ffn", "n_pre", "n_core", "n_coda", "k_max",
        "max_batch", "max_prefix", "max_block", "max_prefill_rows", "mask_id", "dtype")] + \
        [("rms_eps", c_float), ("rope_theta", c_float), ("depth_on_demand", c_int32), ("kv_dtype", c_int32),
         ("cache_depths", c_int32), ("weight_row_pad", c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("attn_norm", "wqkv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate_up",
                                        "w_down")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("final_norm", c_void_p), ("exit_w", c_void_p),
                ("exit_b", c_float), ("layers", POINTER(LayerWeights))]


class StepArgs(ctypes.Structure):
    _fields_ = [("batch", c_int32), ("block_len", c_int32), ("block_ids", c_void_p), ("tau_ent", c_float),
                ("tau_halt", c_float), ("k_loops", c_int32), ("flags", c_uint32), ("boost_tok", c_void_p),
                ("boost_val", c_void_p), ("tf_commit_loop", c_void_p), ("tf_tokens", c_void_p),
                ("tf_stop_loop", c_void_p), ("sample_seed", c_uint64), ("sample_step", c_uint32)]


class StepOut(ctypes.Structure):
    _fields_ = [("tokens", c_void_p), ("commit_loop", c_void_p), ("loops", c_void_p), ("entropy", c_void_p),
                ("lam", c_void_p), ("halt", c_void_p), ("lse", c_void_p), ("argmax", c_void_p),
                ("hidden", c_void_p), ("n_committed", c_int32), ("loops_run", c_int32), ("sampled", c_void_p)]


class BlockArgs(ctypes.Structure):
    _fields_ = [("step", StepArgs), ("max_steps", c_int32), ("append", c_int32), ("deepen", c_int32)]


class BlockOut(ctypes.Structure):
    _fields_ = [("tokens", c_void_p), ("commit_step", c_void_p), ("commit_loop", c_void_p), ("n_steps", c_int32),
                ("n_committed", c_int32), ("built_depth", c_int32)]


class AlodlmError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("alodlm error %d: %s" % (code, msg))
        self.code = code


_lib = None


def load(path: str = LIB_PATH):
    """Loads the HIP library; raises if it is missing (build it with __graft_entry__.build())."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("HIP library %s is not built; run __graft_entry__.build() first" % path)
    lib = ctypes.CDLL(path)
    P = POINTER
    lib.alodlm_workspace_bytes.argtypes = [P(Config), P(c_size_t)]
    lib.alodlm_kv_slots.argtypes = [P(Config), P(c_int32)]
    lib.alodlm_create.argtypes = [P(Config), P(Weights), c_void_p, c_size_t, c_void_p, P(c_void_p)]
    lib.alodlm_prefill_kv.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p]
    lib.alodlm_prefill_kv_synthetic.argtypes = [c_void_p, c_int32, c_int32, c_uint32, c_float, c_float, c_void_p]
    lib.alodlm_denoise_step.argtypes = [c_void_p, P(StepArgs), P(StepOut)]
    lib.alodlm_extend_kv.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_void_p]
    lib.alodlm_prefill_kv_depth.argtypes = [c_void_p, c_int32, c_int32, c_void_p, c_int32]
    lib.alodlm_deepen_kv.argtypes = [c_void_p, c_int32]
    lib.alodlm_denoise_block.argtypes = [c_void_p, P(BlockArgs), P(BlockOut)]
    lib.alodlm_readout_commit.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_float, c_float, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p]
    lib.alodlm_readout_commit_static.argtypes = lib.alodlm_readout_commit.argtypes
    lib.alodlm_last_step_stats.argtypes = [c_void_p, P(c_int64), P(c_int32)]
    lib.alodlm_last_error.argtypes = [c_void_p]
    lib.alodlm_last_error.restype = c_char_p
    lib.alodlm_destroy.argtypes = [c_void_p]
    lib.alodlm_destroy.restype = None
    lib.alodlm_synth_fill.argtypes = [c_void_p, c_int32, c_uint64, c_uint64, c_uint32, c_uint32, c_float, c_float,
                                      c_void_p]
    lib.alodlm_diag_gemm.argtypes = [c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_int32, c_int32, c_int32, c_void_p]
    lib.alodlm_diag_readout_sample.argtypes = [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_uint64,
                                               c_uint32, c_uint32, c_void_p, c_void_p, c_size_t, c_int32, c_int32,
                                               c_void_p]
    lib.alodlm_diag_gemm_choice.argtypes = [c_int32, c_int32, c_int32, c_int32, c_size_t, P(c_int32), P(c_int32),
                                            c_char_p, c_size_t]
    lib.alodlm_diag_timing_enable.argtypes = [c_void_p, c_int32]
    lib.alodlm_diag_buffer_offset.argtypes = [c_void_p, ctypes.c_char_p]
    lib.alodlm_diag_buffer_offset.restype = c_int64
    lib.alodlm_diag_read_kv.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p]
    lib.alodlm_diag_timing_read.argtypes = [c_void_p, c_int32, POINTER(ctypes.c_double), POINTER(c_int64)]
    for name in EXPORTS:
        if name not in ("alodlm_last_error", "alodlm_destroy", "alodlm_diag_buffer_offset"):
            getattr(lib, name).restype = c_int32
    _lib = lib
    return lib


def _check(rc: int, ctx=None):
    if rc != OK:
        msg = load().alodlm_last_error(ctx)
        raise AlodlmError(rc, msg.decode() if msg else "")


def workspace_bytes(cfg: Config) -> int:
    n = c_size_t(0)
    _check(load().alodlm_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def kv_slots(cfg: Config) -> int:
    n = c_int32(0)
    _check(load().alodlm_kv_slots(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def create(cfg: Config, weights: Weights, workspace_ptr: int, ws_bytes: int, stream_ptr: int) -> int:
    out = c_void_p(0)
    _check(load().alodlm_create(ctypes.byref(cfg), ctypes.byref(weights), c_void_p(workspace_ptr), ws_bytes,
                                c_void_p(stream_ptr), ctypes.byref(out)))
    return out.value


def prefill_kv(ctx: int, batch: int, prefix_len: int, prefix_ids_ptr: int, avail_ptr: int = 0):
    _check(load().alodlm_prefill_kv(c_void_p(ctx), batch, prefix_len, c_void_p(prefix_ids_ptr),
                                    c_void_p(avail_ptr or None)), c_void_p(ctx))


def prefill_kv_synthetic(ctx: int, batch: int, prefix_len: int, seed: int, k_scale: float, v_scale: float,
                         avail_ptr: int = 0):
    _check(load().alodlm_prefill_kv_synthetic(c_void_p(ctx), batch, prefix_len, seed, k_scale, v_scale,
                                              c_void_p(avail_ptr or None)), c_void_p(ctx))


def denoise_step(ctx: int, args: StepArgs, out: StepOut):
    _check(load().alodlm_denoise_step(c_void_p(ctx), ctypes.byref(args), ctypes.byref(out)), c_void_p(ctx))


def prefill_kv_depth(ctx: int, batch: int, prefix_len: int, prefix_ids_ptr: int, depth: int):
    _check(load().alodlm_prefill_kv_depth(c_void_p(ctx), batch, prefix_len, c_void_p(prefix_ids_ptr), depth),
           c_void_p(ctx))


def deepen_kv(ctx: int, depth: int):
    _check(load().alodlm_deepen_kv(c_void_p(ctx), depth), c_void_p(ctx))


def extend_kv(ctx: int, batch: int, n_new: int, new_ids_ptr: int, avail_ptr: int = 0):
    _check(load().alodlm_extend_kv(c_void_p(ctx), batch, n_new, c_void_p(new_ids_ptr), c_void_p(avail_ptr or None)),
           c_void_p(ctx))


def denoise_block(ctx: int, args: BlockArgs, out: BlockOut):
    _check(load().alodlm_denoise_block(c_void_p(ctx), ctypes.byref(args), ctypes.byref(out)), c_void_p(ctx))


def readout_commit(ctx: int, rows_ptr: int, n_rows: int, group: int, tau_ent: float, tau_halt: float,
                   boost_tok_ptr: int, boost_val_ptr: int, entropy: int, lse: int, lam: int, halt: int, argmax: int,
                   tokens: int, commit_loop: int, embed_out: int):
    _check(load().alodlm_readout_commit(c_void_p(ctx), c_void_p(rows_ptr), n_rows, group, tau_ent, tau_halt,
                                        c_void_p(boost_tok_ptr or None), c_void_p(boost_val_ptr or None),
                                        c_void_p(entropy), c_void_p(lse), c_void_p(lam), c_void_p(halt),
                                        c_void_p(argmax), c_void_p(tokens), c_void_p(commit_loop),
                                        c_void_p(embed_out)), c_void_p(ctx))


def readout_commit_static(ctx: int, rows_ptr: int, n_rows: int, group: int, tau_ent: float, tau_halt: float,
                          boost_tok_ptr: int, boost_val_ptr: int, entropy: int, lse: int, lam: int, halt: int,
                          argmax: int, tokens: int, commit_loop: int, embed_out: int):
    _check(load().alodlm_readout_commit_static(c_void_p(ctx), c_void_p(rows_ptr), n_rows, group, tau_ent, tau_halt,
                                               c_void_p(boost_tok_ptr or None), c_void_p(boost_val_ptr or None),
                                               c_void_p(entropy), c_void_p(lse), c_void_p(lam), c_void_p(halt),
                                               c_void_p(argmax), c_void_p(tokens), c_void_p(commit_loop),
                                               c_void_p(embed_out)), c_void_p(ctx))


def last_step_stats(ctx: int):
    calls, loops = c_int64(0), c_int32(0)
    _check(load().alodlm_last_step_stats(c_void_p(ctx), ctypes.byref(calls), ctypes.byref(loops)), c_void_p(ctx))
    return calls.value, loops.value


def destroy(ctx: int):
    if ctx:
        load().alodlm_destroy(c_void_p(ctx))


def synth_fill(dst_ptr: int, dtype: int, start: int, n: int, seed: int, tensor: int, scale: float, offset: float,
               stream_ptr: int):
    rc = load().alodlm_synth_fill(c_void_p(dst_ptr), dtype, start, n, seed, tensor, scale, offset,
                                  c_void_p(stream_ptr))
    if rc != 0:
        raise AlodlmError(rc, "alodlm_synth_fill failed")


def diag_gemm(epi: int, M: int, N: int, K: int, A_ptr: int, B_ptr: int, C_ptr: int, act_ptr: int, scratch_ptr: int,
              scratch_floats: int, force_splits: int, force_generic: int, stream_ptr: int, force_tile: int = -1):
    rc = load().alodlm_diag_gemm(epi, M, N, K, c_void_p(A_ptr), c_void_p(B_ptr), c_void_p(C_ptr or None),
                                 c_void_p(act_ptr or None), c_void_p(scratch_ptr or None), scratch_floats,
                                 force_splits, force_generic, force_tile, c_void_p(stream_ptr))
    if rc != 0:
        raise AlodlmError(rc, "alodlm_diag_gemm failed")


def diag_readout_sample(M: int, N: int, K: int, A_ptr: int, B_ptr: int, row_key_ptr: int, seed: int, c2: int, c3: int,
                        tok_ptr: int, scratch_ptr: int, scratch_floats: int, force_generic: int, stream_ptr: int,
                        force_tile: int = -1):
    rc = load().alodlm_diag_readout_sample(M, N, K, c_void_p(A_ptr), c_void_p(B_ptr), c_void_p(row_key_ptr), seed, c2,
                                           c3, c_void_p(tok_ptr), c_void_p(scratch_ptr), scratch_floats,
                                           force_generic, force_tile, c_void_p(stream_ptr))
    if rc != 0:
        raise AlodlmError(rc, "alodlm_diag_readout_sample failed")


def gemm_choice(epi: int, M: int, N: int, K: int, scratch_floats: int):
    """(tile, split-K, kernel name) the matrix-core dispatcher takes for the shape."""
    t, sp = c_int32(0), c_int32(0)
    buf = ctypes.create_string_buffer(256)
    rc = load().alodlm_diag_gemm_choice(epi, M, N, K, scratch_floats, ctypes.byref(t), ctypes.byref(sp), buf, 256)
    if rc != 0:
        raise AlodlmError(rc, "alodlm_diag_gemm_choice: shape not taken by the matrix cores")
    return t.value, sp.value, buf.value.decode()


def timing_enable(ctx: int, on: bool):
    _check(load().alodlm_diag_timing_enable(c_void_p(ctx), 1 if on else 0), c_void_p(ctx))


def timing_read(ctx: int) -> dict:
    out = {}
    for k, name in enumerate(K_CLASSES):
        ms, n = ctypes.c_double(0), c_int64(0)
        _check(load().alodlm_diag_timing_read(c_void_p(ctx), k, ctypes.byref(ms), ctypes.byref(n)), c_void_p(ctx))
        out[name] = (ms.value, n.value)
    return out


def read_kv(ctx: int, slot: int, b: int, j0: int, n: int, dst_k_ptr: int, dst_v_ptr: int):
    rc = load().alodlm_diag_read_kv(c_void_p(ctx), slot, b, j0, n, c_void_p(dst_k_ptr), c_void_p(dst_v_ptr))
    if rc != 0:
        raise AlodlmError(rc, "alodlm_diag_read_kv failed")


def buffer_offset(ctx: int, name: str) -> int:
    return load().alodlm_diag_buffer_offset(c_void_p(ctx), name.encode())
