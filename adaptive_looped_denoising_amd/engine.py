"""Python-side driver of the HIP library for a seeded workload.

PyTorch provides device memory and the stream; every computation of the step
runs in libalodlm.so through the ctypes binding.  Weights are uploaded from the
host generator for small models and filled on the device (same counter-based
definition) for large ones.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B
from . import synth


def _dev_tensor_from_storage(arr: np.ndarray, device) -> torch.Tensor:
    """Upload a host array in storage format (uint16 bf16 bits or float32)."""
    if arr.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


# linear weights the library reads with a row pitch of in + weight_row_pad elements
PADDED = ("wqkv", "wo", "w_gate_up", "w_down", "lm_head")
# Default pad of bf16 models: dense 4096-wide bf16 rows are 8 KB apart, which puts the same column
# of every row a matrix tile streams on the same memory channels; this pad staggers them.
DEFAULT_WEIGHT_ROW_PAD = 64


def _ptr(t: Optional[torch.Tensor]) -> int:
    return 0 if t is None else t.data_ptr()


@dataclass
class StepResult:
    tokens: np.ndarray
    commit_loop: np.ndarray
    loops: np.ndarray
    n_committed: int
    loops_run: int
    entropy: Optional[np.ndarray] = None
    lam: Optional[np.ndarray] = None
    halt: Optional[np.ndarray] = None
    lse: Optional[np.ndarray] = None
    argmax: Optional[np.ndarray] = None
    sampled: Optional[np.ndarray] = None
    hidden: Optional[np.ndarray] = None


class Engine:
    def __init__(self, w: synth.Workload, device: str = "cuda", weight_source: Optional[str] = None,
                 max_prefill_rows: Optional[int] = None, overrides: Optional[Dict[str, np.ndarray]] = None,
                 exit_b: Optional[float] = None, max_prefix: Optional[int] = None, depth_on_demand: bool = False,
                 weight_row_pad: Optional[int] = None):
        """``max_prefix``: cache capacity per sequence (default the workload's prefix; larger to
        append blocks).  ``depth_on_demand``: keep the prefix state for depth-by-depth builds.
        ``weight_row_pad``: elements after every row of the linear weights (default
        DEFAULT_WEIGHT_ROW_PAD for bf16 models, 0 for fp32)."""
        self.lib = B.load()
        self.w = w
        self.device = torch.device(device)
        self.stream = torch.cuda.current_stream(self.device)
        D = w.dims
        self.tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.cdtype = B.DTYPE_BF16 if w.dtype == "bf16" else B.DTYPE_FP32
        specs = synth.weight_specs(w)
        n_params = sum(int(np.prod(s["shape"])) for s in specs)
        if weight_source is None:
            weight_source = "host" if n_params < 50_000_000 else "device"
        if weight_row_pad is None:
            weight_row_pad = DEFAULT_WEIGHT_ROW_PAD if w.dtype == "bf16" else 0
        self.weight_row_pad = weight_row_pad
        self.tensors: Dict[str, torch.Tensor] = {}
        for s in specs:
            name = s["name"]
            if overrides and name in overrides:
                t = _dev_tensor_from_storage(overrides[name], self.device)
            elif weight_source == "host":
                t = _dev_tensor_from_storage(synth.gen_tensor(s, w.seed, w.dtype), self.device)
            else:
                t = torch.empty(s["shape"], dtype=self.tdtype, device=self.device)
                if "const" in s:
                    B.synth_fill(t.data_ptr(), self.cdtype, 0, t.numel(), 0, 0, 0.0, float(s["const"]),
                                 self.stream.cuda_stream)
                else:
                    B.synth_fill(t.data_ptr(), self.cdtype, 0, t.numel(), w.seed, s["tensor"], float(s["scale"]),
                                 0.0, self.stream.cuda_stream)
            if weight_row_pad and name.split(".")[-1] in PADDED:
                # the library reads these [out][in] with a row pitch of in + weight_row_pad
                p = torch.zeros((t.shape[0], t.shape[1] + weight_row_pad), dtype=t.dtype, device=self.device)
                p[:, :t.shape[1]] = t
                del t
                t = p
            self.tensors[name] = t
        self.cfg = B.Config(
            vocab=D.vocab, d_model=D.d_model, n_q_heads=D.n_q_heads, n_kv_heads=D.n_kv_heads, head_dim=D.head_dim,
            ffn=D.ffn, n_pre=D.n_pre, n_core=D.n_core, n_coda=D.n_coda, k_max=w.k_max, max_batch=w.batch,
            max_prefix=max(w.prefix, max_prefix or 0), max_block=w.block,
            max_prefill_rows=max_prefill_rows if max_prefill_rows is not None else min(
                w.batch * max(w.prefix, max_prefix or 0), max(w.prefix, max_prefix or 0, 8192)),
            mask_id=w.mask_id, dtype=self.cdtype, rms_eps=w.rms_eps, rope_theta=w.rope_theta,
            depth_on_demand=1 if depth_on_demand else 0, kv_dtype=B.KV_FP8 if w.kv_dtype == "fp8" else B.KV_SAME,
            cache_depths=w.cache_depths, weight_row_pad=weight_row_pad)
        nl = D.n_layers
        self.layer_arr = (B.LayerWeights * max(nl, 1))()
        for l in range(nl):
            p = "layers.%d." % l
            lw = self.layer_arr[l]
            for f in ("attn_norm", "wqkv", "q_norm", "k_norm", "wo", "ffn_norm", "w_gate_up", "w_down"):
                setattr(lw, f, self.tensors[p + f].data_ptr())
        self.exit_b = w.exit_bias() if exit_b is None else float(exit_b)
        self.weights = B.Weights(embed=self.tensors["embed"].data_ptr(), lm_head=self.tensors["lm_head"].data_ptr(),
                                 final_norm=self.tensors["final_norm"].data_ptr(),
                                 exit_w=self.tensors["exit_w"].data_ptr(), exit_b=self.exit_b,
                                 layers=self.layer_arr)
        self.ws_bytes = B.workspace_bytes(self.cfg)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        base = self.ws.data_ptr()
        self.ws_ptr = (base + 255) & ~255
        self.ctx = B.create(self.cfg, self.weights, self.ws_ptr, self.ws_bytes, self.stream.cuda_stream)
        self.kv_slots = B.kv_slots(self.cfg)
        # step inputs
        self.block_ids = torch.from_numpy(synth.block_ids(w)).to(self.device)
        bt, bv = synth.boosts(w)
        self.boost_tok = torch.from_numpy(bt).to(self.device)
        self.boost_val = torch.from_numpy(bv).to(self.device)
        self.avail = torch.from_numpy(synth.avail_depth(w)).to(self.device) if w.prefix else None
        Bn, L = w.batch, w.block
        self.out_tokens = torch.empty((Bn, L), dtype=torch.int32, device=self.device)
        self.out_cl = torch.empty((Bn, L), dtype=torch.int8, device=self.device)
        self.out_loops = torch.empty((Bn,), dtype=torch.int8, device=self.device)

    # ------------------------------------------------------------------ prefix cache
    def prefill(self, prefix_ids: Optional[np.ndarray] = None, depth: Optional[int] = None):
        """Builds the prefix cache; ``depth``: depth-on-demand build to that Core depth."""
        w = self.w
        av = _ptr(self.avail)
        if depth is not None:
            ids = synth.prefix_ids(w) if prefix_ids is None else prefix_ids
            self.prefix_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(self.device)
            B.prefill_kv_depth(self.ctx, w.batch, w.prefix, _ptr(self.prefix_ids) if w.prefix else 0, depth)
        elif w.kv == "synthetic":
            ks, vs = synth.synthetic_kv_scales(w)
            B.prefill_kv_synthetic(self.ctx, w.batch, w.prefix, w.seed, float(np.float32(ks)), float(np.float32(vs)),
                                   av)
        else:
            ids = synth.prefix_ids(w) if prefix_ids is None else prefix_ids
            self.prefix_ids = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).to(self.device)
            B.prefill_kv(self.ctx, w.batch, w.prefix, _ptr(self.prefix_ids) if w.prefix else 0, av)
        torch.cuda.synchronize(self.device)

    # ------------------------------------------------------------------ step
    def make_args(self, tau_ent=None, tau_halt=None, k_loops=None, boost=True, teacher=None, block_ids=None,
                  sample=None):
        """``sample``: {"seed", "step"} commits Gumbel-max draws (ALODLM_STEP_SAMPLE)."""
        w = self.w
        if block_ids is not None:
            self.block_ids = torch.from_numpy(np.ascontiguousarray(block_ids, dtype=np.int32)).to(self.device)
        args = B.StepArgs(batch=w.batch, block_len=w.block, block_ids=_ptr(self.block_ids),
                          tau_ent=w.tau_ent if tau_ent is None else tau_ent,
                          tau_halt=w.tau_halt if tau_halt is None else tau_halt,
                          k_loops=w.k_max if k_loops is None else k_loops, flags=0,
                          boost_tok=_ptr(self.boost_tok) if boost else 0,
                          boost_val=_ptr(self.boost_val) if boost else 0)
        if teacher is not None:
            Bn, L = w.batch, w.block
            cl = np.zeros((Bn, L), dtype=np.int8)
            tk = np.zeros((Bn, L), dtype=np.int32)
            sl = np.zeros((Bn,), dtype=np.int8)
            for b, t in teacher.items():
                cl[b] = t["commit_loop"]
                tk[b] = t["tokens"]
                sl[b] = t["stop_loop"]
            self._tf = [torch.from_numpy(x).to(self.device) for x in (cl, tk, sl)]
            args.flags = B.STEP_TEACHER_FORCED
            args.tf_commit_loop, args.tf_tokens, args.tf_stop_loop = (t.data_ptr() for t in self._tf)
        if sample is not None:
            args.flags |= B.STEP_SAMPLE
            args.sample_seed = int(sample["seed"])
            args.sample_step = int(sample["step"])
        return args

    def make_out(self, k_loops: int, records: bool = False, hidden: bool = False, sampled: bool = False):
        w = self.w
        out = B.StepOut(tokens=_ptr(self.out_tokens), commit_loop=_ptr(self.out_cl), loops=_ptr(self.out_loops))
        self._rec = None
        if records:
            shp = (k_loops, w.batch, w.block)
            self._rec = dict(entropy=torch.empty(shp, dtype=torch.float32, device=self.device),
                             lam=torch.empty(shp, dtype=torch.float32, device=self.device),
                             halt=torch.empty(shp, dtype=torch.float32, device=self.device),
                             lse=torch.empty(shp, dtype=torch.float32, device=self.device),
                             argmax=torch.empty(shp, dtype=torch.int32, device=self.device))
            if sampled:
                self._rec["sampled"] = torch.empty(shp, dtype=torch.int32, device=self.device)
            for k, t in self._rec.items():
                setattr(out, k, t.data_ptr())
        self._hidden = None
        if hidden:
            self._hidden = torch.full((k_loops, w.batch, w.block, w.dims.d_model), float("nan"), dtype=torch.float32,
                                      device=self.device)
            out.hidden = self._hidden.data_ptr()
        return out

    def run(self, args: B.StepArgs, out: B.StepOut):
        B.denoise_step(self.ctx, args, out)

    def step(self, tau_ent=None, tau_halt=None, k_loops=None, boost=True, teacher=None, records=False,
             hidden=False, block_ids=None, sample=None) -> StepResult:
        args = self.make_args(tau_ent, tau_halt, k_loops, boost, teacher, block_ids, sample)
        out = self.make_out(args.k_loops, records, hidden, sampled=sample is not None)
        self.run(args, out)
        torch.cuda.synchronize(self.device)
        res = StepResult(tokens=self.out_tokens.cpu().numpy(), commit_loop=self.out_cl.cpu().numpy(),
                         loops=self.out_loops.cpu().numpy(), n_committed=out.n_committed, loops_run=out.loops_run)
        if self._rec is not None:
            for k, t in self._rec.items():
                setattr(res, k, t.cpu().numpy())
        if self._hidden is not None:
            res.hidden = self._hidden.cpu().numpy()
        return res

    def deepen(self, depth: int):
        B.deepen_kv(self.ctx, depth)
        torch.cuda.synchronize(self.device)

    # ------------------------------------------------------------------ outer loop, cache growth
    def extend(self, new_ids: np.ndarray, avail: Optional[np.ndarray] = None):
        """Appends positions (ids [batch][n]) to every sequence's prefix cache."""
        ids = torch.from_numpy(np.ascontiguousarray(new_ids, dtype=np.int32)).to(self.device)
        av = None if avail is None else torch.from_numpy(np.ascontiguousarray(avail, dtype=np.uint8)).to(self.device)
        B.extend_kv(self.ctx, ids.shape[0], ids.shape[1], ids.data_ptr(), _ptr(av))
        torch.cuda.synchronize(self.device)

    def make_block(self, tau_ent=None, tau_halt=None, k_loops=None, boost=True, block_ids=None, sample=None,
                   max_steps=0, append=False, deepen=False):
        w = self.w
        step = self.make_args(tau_ent, tau_halt, k_loops, boost, None, block_ids, sample)
        args = B.BlockArgs(step=step, max_steps=max_steps, append=1 if append else 0, deepen=1 if deepen else 0)
        self._blk = dict(tokens=torch.empty((w.batch, w.block), dtype=torch.int32, device=self.device),
                         commit_step=torch.empty((w.batch, w.block), dtype=torch.int16, device=self.device),
                         commit_loop=torch.empty((w.batch, w.block), dtype=torch.int8, device=self.device))
        out = B.BlockOut(tokens=self._blk["tokens"].data_ptr(), commit_step=self._blk["commit_step"].data_ptr(),
                         commit_loop=self._blk["commit_loop"].data_ptr())
        return args, out

    def denoise_block(self, **kw) -> dict:
        """Outer loop: steps until no mask in the block (``sample`` = {"seed", "step"}: first step's
        counter); returns final tokens, per-position commit step and loop, steps and commits."""
        args, out = self.make_block(**kw)
        B.denoise_block(self.ctx, args, out)
        torch.cuda.synchronize(self.device)
        res = {k: v.cpu().numpy() for k, v in self._blk.items()}
        res.update(n_steps=out.n_steps, n_committed=out.n_committed, built_depth=out.built_depth)
        return res

    def read_kv(self, slot: int, b: int, j0: int, n: int):
        """K and V rows of one cache slot and sequence, as float32 numpy arrays [Hkv][n][hd] (fp8
        storage decoded by torch's float8_e4m3fn)."""
        D = self.w.dims
        kdt = torch.float8_e4m3fn if self.w.kv_dtype == "fp8" else self.tdtype
        k = torch.empty((D.n_kv_heads, n, D.head_dim), dtype=kdt, device=self.device)
        v = torch.empty_like(k)
        B.read_kv(self.ctx, slot, b, j0, n, k.data_ptr(), v.data_ptr())
        torch.cuda.synchronize(self.device)
        return k.cpu().float().numpy(), v.cpu().float().numpy()

    def stats(self):
        return B.last_step_stats(self.ctx)

    # ------------------------------------------------------------------ readout half of a loop
    def readout_commit(self, rows: torch.Tensor, group: int, tau_ent: float, tau_halt: float,
                       boost_tok: Optional[torch.Tensor] = None, boost_val: Optional[torch.Tensor] = None,
                       static_scratch: bool = False, out: Optional[dict] = None) -> dict:
        """``static_scratch``: the allocation-free entry point (scratch in the library's fixed array).
        ``out``: the output tensors of an earlier call of the same size, reused."""
        n = rows.shape[0]
        dev = self.device
        o = out if out is not None else dict(entropy=torch.empty(n, dtype=torch.float32, device=dev),
                 lse=torch.empty(n, dtype=torch.float32, device=dev),
                 lam=torch.empty(n, dtype=torch.float32, device=dev),
                 halt=torch.empty(n, dtype=torch.float32, device=dev),
                 argmax=torch.empty(n, dtype=torch.int32, device=dev),
                 tokens=torch.empty(n, dtype=torch.int32, device=dev),
                 commit_loop=torch.empty(n, dtype=torch.int8, device=dev),
                 embed=torch.empty((n, self.w.dims.d_model), dtype=torch.float32, device=dev))
        fn = B.readout_commit_static if static_scratch else B.readout_commit
        fn(self.ctx, rows.data_ptr(), n, group, tau_ent, tau_halt, _ptr(boost_tok), _ptr(boost_val),
           o["entropy"].data_ptr(), o["lse"].data_ptr(), o["lam"].data_ptr(), o["halt"].data_ptr(),
           o["argmax"].data_ptr(), o["tokens"].data_ptr(), o["commit_loop"].data_ptr(), o["embed"].data_ptr())
        return o

    def close(self):
        if getattr(self, "ctx", 0):
            B.destroy(self.ctx)
            self.ctx = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
