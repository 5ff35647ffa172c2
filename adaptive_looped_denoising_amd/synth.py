"""Seeded synthetic workloads for the ALoDLM looped denoising step.

This module is the input generator shared by the oracle side (tests, the
CPU baseline) and the GPU side (tests, bench).  It holds no arithmetic of the
method: only the workload shapes, the counter-based random draws and the
recipes that turn them into weights, token ids, planted readout boosts,
depth-availability maps and synthetic prefix K/V.

Every tensor is a pure function of (seed, tensor id, element index) through
Philox4x32-10 (Salmon et al., SC'11); see ``synth_host.c`` for the value maps.
Normal-looking values use the Irwin-Hall sum of four 16-bit uniforms scaled in
one fp32 multiply, so the GPU library's own generator reproduces them bit for
bit and the largest tensors never have to cross PCIe.

Workload shapes follow the ALoDLM summary page (arXiv 2610.04198 summary,
sections "Core method" and "Experiments": Qwen3 backbones, K = 4 loops,
8B split Prelude [0,10) / Core [10,26) / Coda [26,36), tau sweep, 16/32-token
windows) and the explainer page's measured first-pass halting mean of 0.417.
"""
from __future__ import annotations

import ctypes
import json
import math
import os
import subprocess
from dataclasses import dataclass, replace
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SRC = os.path.join(_HERE, "synth_host.c")
_HOST_LIB = os.path.join(_HERE, "_synth_host.so")

IH4_STD = math.sqrt((65536.0 ** 2 - 1.0) / 3.0)  # std of the Irwin-Hall(4) integer draw

# Tensor ids (the second Philox key word).
T_EMBED = 1
T_LMHEAD = 2
T_EXITW = 4
T_PREFIX_IDS = 10
T_EASY_PERM = 11
T_BOOST_TOK = 12
T_BOOST_VAL = 13
T_ROWS = 14
T_AVAIL_PERM = 15
T_LAYER_BASE = 256  # + 16 * layer + part
P_WQKV, P_WO, P_WGU, P_WDOWN = 1, 4, 6, 7
T_KV_BASE = 0x10000  # + 2 * slot (+1 for V)


def layer_tensor(layer: int, part: int) -> int:
    return T_LAYER_BASE + 16 * layer + part


def kv_tensor(slot: int, is_v: bool) -> int:
    return T_KV_BASE + 2 * slot + (1 if is_v else 0)


# ---------------------------------------------------------------------------
# host generator (C, built with gcc on first use)
# ---------------------------------------------------------------------------
_lib = None


def build_host_lib(force: bool = False) -> str:
    if force or not os.path.exists(_HOST_LIB) or os.path.getmtime(_HOST_LIB) < os.path.getmtime(_HOST_SRC):
        tmp = _HOST_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                               _HOST_SRC, "-o", tmp])
        os.replace(tmp, _HOST_LIB)
    return _HOST_LIB


def _host():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build_host_lib())
        u64, u32, vp, f32 = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_float
        lib.alodlm_synth_ih4_f32.argtypes = [vp, u64, u64, u32, u32, f32]
        lib.alodlm_synth_ih4_bf16.argtypes = [vp, u64, u64, u32, u32, f32]
        lib.alodlm_synth_u32.argtypes = [vp, u64, u64, u32, u32]
        lib.alodlm_synth_philox4x32_10.argtypes = [vp, vp, vp]
        _lib = lib
    return _lib


def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    _host().alodlm_synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def u32(n: int, seed: int, tensor: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    if n:
        _host().alodlm_synth_u32(out.ctypes.data, start, n, seed, tensor)
    return out


def ih4(shape, seed: int, tensor: int, scale: float, dtype: str, start: int = 0) -> np.ndarray:
    """Irwin-Hall(4) draws times ``scale``: float32 array, or uint16 bfloat16 bits."""
    n = int(np.prod(shape)) if len(shape) else 1
    if dtype == "bf16":
        out = np.empty(n, dtype=np.uint16)
        if n:
            _host().alodlm_synth_ih4_bf16(out.ctypes.data, start, n, seed, tensor, float(np.float32(scale)))
    else:
        out = np.empty(n, dtype=np.float32)
        if n:
            _host().alodlm_synth_ih4_f32(out.ctypes.data, start, n, seed, tensor, float(np.float32(scale)))
    return out.reshape(shape)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest even); returns the uint16 bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def as_f32(a: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Dims:
    vocab: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    n_pre: int
    n_core: int
    n_coda: int

    @property
    def n_layers(self) -> int:
        return self.n_pre + self.n_core + self.n_coda

    @property
    def qkv_out(self) -> int:
        return (self.n_q_heads + 2 * self.n_kv_heads) * self.head_dim

    def kv_slots(self, k_max: int) -> int:
        return self.n_pre + self.n_core * k_max + self.n_coda


@dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    dtype: str          # "fp32" | "bf16"
    batch: int
    prefix: int
    block: int
    k_max: int          # loop cap K (and the number of Core depth planes in the cache)
    tau_ent: float      # entropy threshold in nats (commit iff H <= tau_ent)
    tau_halt: float     # halting threshold q on the mean cumulative halt of unresolved rows
    seed: int
    boost_lo: float = 4.0
    boost_hi: float = 10.0
    easy_frac: float = 0.6
    kv: str = "prefill"     # "prefill": computed from prefix ids; "synthetic": Philox K/V
    short_frac: float = 0.0  # fraction of prefix positions whose cache stops at short_depth
    short_depth: int = 0
    kv_dtype: str = "same"  # K/V storage: "same" (the model dtype) or "fp8" (OCP E4M3)
    cache_depths: int = 0   # Core depths kept in the cache (0: all k_max)
    weight_std: float = 0.02
    halt_target: float = 0.42
    rms_eps: float = 1e-6
    rope_theta: float = 1.0e6

    @property
    def mask_id(self) -> int:
        return self.dims.vocab - 1

    @property
    def weight_scale(self) -> float:
        return self.weight_std / IH4_STD

    @property
    def n_easy(self) -> int:
        return int(math.floor(self.easy_frac * self.block + 0.5))

    def exit_bias(self) -> float:
        """ExitGate bias so that the mean first-loop halt probability is about halt_target.

        The named workloads take the bias stored in exit_bias.json, solved on the realised loop-1
        readout of their seeded inputs (mean over block rows of sigmoid(w_g . r + b) = 0.42) by the
        oracle-only script oracle/calibrate_exit_bias.py; the table entry is used only for the
        inputs it was solved on.  Any other workload (test variants) takes a closed form: a
        readout row r has unit RMS, so w_g . r spreads as N(0, s^2) with s = weight_std * sqrt(d),
        and the bias solves E[sigmoid(b + s Z)] = target with the probit approximation of the
        logistic-normal integral (MacKay 1992): b = logit(target) * sqrt(1 + pi s^2 / 8).
        """
        ent = _bias_table().get(self.name)
        if ent is not None and ent.get("inputs") == bias_fingerprint(self) and self.halt_target == _BIAS_TARGET[0]:
            return float(np.float32(ent["exit_b"]))
        s = self.weight_std * math.sqrt(self.dims.d_model)
        t = self.halt_target
        return float(np.float32(math.log(t / (1.0 - t)) * math.sqrt(1.0 + math.pi * s * s / 8.0)))


_BIAS_PATH = os.path.join(_HERE, "exit_bias.json")
_BIAS = None
_BIAS_TARGET = [None]


def _bias_table() -> dict:
    global _BIAS
    if _BIAS is None:
        _BIAS = {}
        if os.path.exists(_BIAS_PATH):
            with open(_BIAS_PATH) as f:
                data = json.load(f)
            _BIAS = data.get("bias", {})
            _BIAS_TARGET[0] = data.get("target")
    return _BIAS


def bias_fingerprint(w: "Workload") -> dict:
    """The inputs a stored ExitGate bias was solved on (everything the loop-1 readout depends on)."""
    return dict(dims=[w.dims.vocab, w.dims.d_model, w.dims.n_q_heads, w.dims.n_kv_heads, w.dims.head_dim,
                      w.dims.ffn, w.dims.n_pre, w.dims.n_core, w.dims.n_coda],
                dtype=w.dtype, seed=w.seed, batch=w.batch, prefix=w.prefix, block=w.block, kv=w.kv,
                short_frac=w.short_frac, short_depth=w.short_depth, kv_dtype=w.kv_dtype,
                weight_std=w.weight_std, rms_eps=w.rms_eps, rope_theta=w.rope_theta)


QWEN3_8B_DIMS = Dims(vocab=151936, d_model=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
                     n_pre=10, n_core=16, n_coda=10)
QWEN3_1P7B_DIMS = Dims(vocab=151936, d_model=2048, n_q_heads=16, n_kv_heads=8, head_dim=128, ffn=6144,
                       n_pre=6, n_core=16, n_coda=6)
TINY_DIMS = Dims(vocab=512, d_model=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=384,
                 n_pre=1, n_core=2, n_coda=1)

WORKLOADS: Dict[str, Workload] = {
    # tiny fp32 step
    "tiny": Workload("tiny", TINY_DIMS, "fp32", batch=1, prefix=32, block=16, k_max=4,
                     tau_ent=0.3, tau_halt=0.5, seed=0),
    # 1.7B-shape step
    "qwen3_1p7b": Workload("qwen3_1p7b", QWEN3_1P7B_DIMS, "bf16", batch=1, prefix=512, block=32, k_max=4,
                           tau_ent=0.6, tau_halt=0.5, seed=2),
    # 8B-shape step (tau swept over 0.1 / 0.6 / 0.9)
    "qwen3_8b": Workload("qwen3_8b", QWEN3_8B_DIMS, "bf16", batch=8, prefix=1024, block=32, k_max=4,
                         tau_ent=0.6, tau_halt=0.5, seed=3),
    # 8B-shape long-context step over a synthetic depth-aware cache
    "qwen3_8b_long": Workload("qwen3_8b_long", QWEN3_8B_DIMS, "bf16", batch=32, prefix=8192, block=64,
                              k_max=6, tau_ent=0.6, tau_halt=0.9, seed=4, kv="synthetic",
                              short_frac=0.25, short_depth=3),
}
TAU_SWEEP_8B = (0.1, 0.6, 0.9)

# Readout + exit microbench at 8B shape (rows stand for post-RMSNorm readout states).
READOUT_ROWS = (32, 256, 2048)
READOUT_SEED = 1
READOUT_GROUP = 32          # rows are grouped into sequences of 32
READOUT_TAU_ENT = 0.6
READOUT_TAU_HALT = 0.5


def workload(name: str, **over) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **over) if over else w


def with_dims(w: Workload, **over) -> Workload:
    return replace(w, dims=replace(w.dims, **over))


# ---------------------------------------------------------------------------
# per-tensor recipes
# ---------------------------------------------------------------------------
def _perm_rank(seed: int, tensor: int, row: int, n: int) -> np.ndarray:
    """Seeded permutation of range(n): positions sorted by a Philox word (ties by position)."""
    words = u32(n, seed, tensor, start=row * n)
    return np.lexsort((np.arange(n), words))


def prefix_ids(w: Workload) -> np.ndarray:
    words = u32(w.batch * w.prefix, w.seed, T_PREFIX_IDS)
    return ((words.astype(np.uint64) * np.uint64(w.dims.vocab)) >> np.uint64(32)).astype(np.int32).reshape(
        w.batch, w.prefix)


def block_ids(w: Workload) -> np.ndarray:
    return np.full((w.batch, w.block), w.mask_id, dtype=np.int32)


def boosts(w: Workload):
    """Planted readout boosts: (tok[B][L] with -1 = none, val[B][L] float32)."""
    B, L, V = w.batch, w.block, w.dims.vocab
    tok = np.full((B, L), -1, dtype=np.int32)
    val = np.zeros((B, L), dtype=np.float32)
    twords = u32(B * L, w.seed, T_BOOST_TOK).reshape(B, L)
    vwords = u32(B * L, w.seed, T_BOOST_VAL).reshape(B, L)
    t_all = ((twords.astype(np.uint64) * np.uint64(V - 1)) >> np.uint64(32)).astype(np.int32)
    frac = (vwords >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)
    v_all = np.float32(w.boost_lo) + np.float32(w.boost_hi - w.boost_lo) * frac
    for b in range(B):
        easy = _perm_rank(w.seed, T_EASY_PERM, b, L)[: w.n_easy]
        tok[b, easy] = t_all[b, easy]
        val[b, easy] = v_all[b, easy]
    return tok, val


def avail_depth(w: Workload) -> np.ndarray:
    """Deepest cached Core depth per prefix position (uint8 [B][P])."""
    B, P = w.batch, w.prefix
    av = np.full((B, P), w.k_max, dtype=np.uint8)
    n_short = int(math.floor(w.short_frac * P + 0.5))
    if n_short:
        for b in range(B):
            av[b, _perm_rank(w.seed, T_AVAIL_PERM, b, P)[:n_short]] = w.short_depth
    return av


def weight_specs(w: Workload) -> List[dict]:
    """Every weight tensor: name, shape, (tensor id, scale) or a constant fill."""
    D = w.dims
    d, hd, F = D.d_model, D.head_dim, D.ffn
    sc = w.weight_scale
    specs = [
        dict(name="embed", shape=(D.vocab, d), tensor=T_EMBED, scale=sc),
        dict(name="lm_head", shape=(D.vocab, d), tensor=T_LMHEAD, scale=sc),
        dict(name="final_norm", shape=(d,), const=1.0),
        dict(name="exit_w", shape=(d,), tensor=T_EXITW, scale=sc),
    ]
    for l in range(D.n_layers):
        p = "layers.%d." % l
        specs += [
            dict(name=p + "attn_norm", shape=(d,), const=1.0),
            dict(name=p + "wqkv", shape=(D.qkv_out, d), tensor=layer_tensor(l, P_WQKV), scale=sc),
            dict(name=p + "q_norm", shape=(hd,), const=1.0),
            dict(name=p + "k_norm", shape=(hd,), const=1.0),
            dict(name=p + "wo", shape=(d, D.n_q_heads * hd), tensor=layer_tensor(l, P_WO), scale=sc),
            dict(name=p + "ffn_norm", shape=(d,), const=1.0),
            dict(name=p + "w_gate_up", shape=(2 * F, d), tensor=layer_tensor(l, P_WGU), scale=sc),
            dict(name=p + "w_down", shape=(d, F), tensor=layer_tensor(l, P_WDOWN), scale=sc),
        ]
    return specs


def gen_tensor(spec: dict, seed: int, dtype: str) -> np.ndarray:
    """Host copy of one weight: uint16 bf16 bits (bf16) or float32 (fp32)."""
    shape = spec["shape"]
    if "const" in spec:
        a = np.full(shape, spec["const"], dtype=np.float32)
        return f32_to_bf16_bits(a).reshape(shape) if dtype == "bf16" else a
    return ih4(shape, seed, spec["tensor"], spec["scale"], dtype)


def host_weights(w: Workload, names: Optional[List[str]] = None) -> Dict[str, np.ndarray]:
    """Host weights in their storage format (uint16 bf16 bits, or float32)."""
    out = {}
    for s in weight_specs(w):
        if names is None or s["name"] in names:
            out[s["name"]] = gen_tensor(s, w.seed, w.dtype)
    return out


def synthetic_kv_scales(w: Workload):
    """(K scale, V scale): K entries of unit spread (post q/k-norm statistics),
    V entries of spread weight_std * sqrt(d) (statistics of W_v applied to a unit-RMS row)."""
    return 1.0 / IH4_STD, w.weight_std * math.sqrt(w.dims.d_model) / IH4_STD


def synthetic_kv_seq(w: Workload, slot: int, b: int, positions: Optional[np.ndarray] = None):
    """Synthetic cache K and V of one (slot, sequence): arrays [Hkv][P'][hd] in storage format.

    Element (b, h, j, e) of a slot is generator index ((b*Hkv + h)*P + j)*hd + e.
    """
    D = w.dims
    Hkv, P, hd = D.n_kv_heads, w.prefix, D.head_dim
    ks, vs = synthetic_kv_scales(w)
    pos = np.arange(P) if positions is None else np.asarray(positions)
    outs = []
    for is_v, sc in ((False, ks), (True, vs)):
        t = kv_tensor(slot, is_v)
        arr = None
        for h in range(Hkv):
            base = ((b * Hkv + h) * P) * hd
            if positions is None:
                blk = ih4((P, hd), w.seed, t, sc, w.dtype, start=base)
            else:
                blk = np.stack([ih4((hd,), w.seed, t, sc, w.dtype, start=base + int(j) * hd) for j in pos])
            if arr is None:
                arr = np.empty((Hkv,) + blk.shape, dtype=blk.dtype)
            arr[h] = blk
        outs.append(arr)
    return outs[0], outs[1]


def readout_rows(n: int, d: int = 4096) -> np.ndarray:
    """Readout microbench rows: unit-spread draws standing for post-RMSNorm states (bf16 bits)."""
    return ih4((n, d), READOUT_SEED, T_ROWS, 1.0 / IH4_STD, "bf16")


def readout_workload(n_rows: int) -> Workload:
    """The readout microbench as a Workload (8B readout shape, one loop, groups of 32 rows)."""
    dims = replace(QWEN3_8B_DIMS, n_pre=0, n_core=1, n_coda=0)   # the heads only need one (unused) layer
    return Workload("readout_%d" % n_rows, dims, "bf16", batch=max(1, n_rows // READOUT_GROUP),
                    prefix=0, block=min(n_rows, READOUT_GROUP), k_max=1, tau_ent=READOUT_TAU_ENT,
                    tau_halt=READOUT_TAU_HALT, seed=READOUT_SEED)
