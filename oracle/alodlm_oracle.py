"""ALoDLM adaptively looped denoising step -- ORACLE (test infrastructure only).

A plain, slow, float64 CPU implementation of what one denoising step of
ALoDLM computes, written from the method pages.  It is test infrastructure:
only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it.  It shares no code with the HIP library and never reads anything
the library produced.

Sources (page titles and sections):
  * "ALoDLM: Adaptively Looped Diffusion Language Models" summary page
    (paper.rainbus.top, arXiv 2610.04198): section "Core method" (Prelude /
    Recurrent Core / Coda split, the two heads, lambda = sigmoid(ExitGate(r)),
    commit iff entropy <= tau, halt when the mean cumulative halt of the
    unresolved positions reaches q, forced exit at s = K, Eq. 3), section
    "Method step details" (Algorithm 1: outer and inner loop, the cumulative
    halting update a <- a + (1 - a) lambda, the forced lowest-entropy commit), section
    "Background" (looped Transformer with shared weights; depth-aware KV
    cache: matching depth first, deepest available as fallback), section
    "Limitations" (the cache holds L + (K-1) m buffers, 84 for 8B at K = 4),
    section "Technical novelty" (10 + 4 x (16 + 10) = 114 layer calls).
  * the tokendh.com explainer of the same paper: entropy and cumulative-halt
    thresholds; committed positions feed back their token embedding.

Readings where the pages are silent (both this oracle and the GPU library
follow them):
  * layer = Qwen3 block: pre-norm RMSNorm, per-head RMSNorm of q and k, RoPE
    (rotate-half pairs (i, i + hd/2), base theta), GQA with q head h reading
    kv head floor(h * Hkv / Hq), softmax scale 1/sqrt(hd), SwiGLU FFN, no biases;
  * the prefix cache is built causally; Core depth d holds the K/V the
    prefix produces on its d-th pass through the Core; Prelude and Coda hold
    one set each, the Coda set computed on the depth-K output;
  * block rows see every prefix key and every block key (no mask); positions
    are 0..P-1 for the prefix and P..P+L-1 for the block;
  * prefix key j is read at depth min(s, d_j) by Core layers in loop s;
  * readout r = final RMSNorm of the Coda output; both heads read r;
  * entropy in nats, commit iff H <= tau_ent; token = argmax, ties to the
    lowest id (greedy decoding) by default; in sampling mode the committed
    token is the draw y ~ p of Algorithm 1 taken by the Gumbel-max rule
    y = argmax_v (z_v + g_v), g_v = -ln(-ln u_v), with u_v from the
    counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
    "Parallel random numbers: as easy as 1, 2, 3", SC'11) at counter
    (v div 4, 64 b + i, s, step), key (seed mod 2^32, seed div 2^32), word
    v mod 4, u = (floor(x / 2^9) + 1/2) / 2^23 (sequence b, block row i,
    loop s); the forced commit takes its row's draw of the last loop too;
    the one-token-per-step mode of the quality tables is tau_ent < 0 (no
    entropy commit, only the forced one);
  * a is updated for positions unresolved at the start of the loop; the halt
    test uses the mean of a over the positions still unresolved after the
    loop's commits, "reaches" meaning >=; every sequence halts on its own;
  * Eq. 3 is applied to every block row that is not unresolved: its state is
    reset to the embedding of its token at the end of every loop;
  * committed rows keep running through every layer as context;
  * if a step committed nothing, the unresolved position of lowest entropy at
    the last loop (ties to the lowest position) commits, recorded as -s_end;
  * ExitGate is a d -> 1 linear map plus sigmoid;
  * a sequence whose block has no masked position runs no loop (loops = 0):
    the outer loop of Algorithm 1 ends once no [MASK] remains;
  * outer loop: denoising steps over a block until no position is masked,
    each step starting from the Prelude of the block with every committed
    token written in; denoising step t (1-based) of a block draws its samples
    with counter word 3 = step0 + t - 1;
  * depth-on-demand prefill (the "Limitations" section's remedy for the
    first-token latency): the prefix is first built to a depth D0 < K, the
    Coda set on the depth-D0 output, every position available at depth D0;
    deepening continues the Core passes from the saved depth-D0 output and
    rebuilds the Coda set on the deeper output (so the result equals a
    prefill built to that depth directly);
  * compressed depth buffers (the "Limitations" section's remedy for the
    memory of the per-depth cache): keys and values -- the cached ones and
    a block's own -- may be stored in the OCP FP8 E4M3 format, rounded once
    from the float32 projection result (nearest, ties to even, saturating
    at +-448); attention then reads those values;
  * a finished block joins the depth-aware cache the way the prefill builds
    it: its positions go through the Prelude once, the Core once per depth
    d = 1..k_max and the Coda once on the depth-k_max output, causally among
    themselves, reading the cached positions as a step does (Core position j
    at depth min(d, avail_j)); they are cached at every depth.  With every
    cached position at full depth this is the prefill of the longer prefix;
  * depth eviction (the "Limitations" section's other memory remedy, dropping
    low-value depth buffers): a cache keeping depths 1..D holds the sets the
    full build computes for the Prelude, the Coda and Core depths 1..D, and
    drops the deeper Core sets; every position's available depth becomes
    min(avail_j, D), so the deepest-available fallback serves deeper loops.
    The value of a depth is taken to fall with the depth (the deeper sets go
    first), since loops past the first few are the rare ones.  A block that
    joins such a cache still runs all k_max Core passes (the Coda set needs
    the depth-k_max output), reading the cached positions at min(d, avail_j),
    and keeps depths 1..D of its own positions.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

F64 = np.float64


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=F64)


def round_bf16(x) -> np.ndarray:
    """Round to bfloat16 the way an fp32 pipeline does: to float32 first, then to the nearest
    bfloat16 (ties to even); returned as float64."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _rnd(x, prec):
    return round_bf16(x) if prec == "bf16" else x


FP8_MAX = 448.0  # largest finite OCP FP8 E4M3 value (1.75 * 2^8)


def round_fp8_e4m3(x) -> np.ndarray:
    """Round to the OCP FP8 E4M3 format (sign, 4 exponent bits with bias 7, 3 fraction bits,
    subnormals, no infinities, largest finite 448) the way a pipeline computing in float32 stores
    it: to float32 first, then to the nearest E4M3 value with ties to even, saturating at +-448.
    Returned as float64."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    a = np.abs(f)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = np.maximum(ex - 1, -6)                # binade exponent; below 2^-6 the subnormal spacing
    q = np.ldexp(1.0, e - 3)                  # spacing of E4M3 values in that binade
    r = np.round(a / q) * q                   # a / q is exact (power-of-two scale); numpy rounds half to even
    r = np.minimum(r, FP8_MAX)
    return np.where(a == 0.0, 0.0, np.copysign(r, f))


def _kv_round(x, prec, kv):
    """Storage rounding of post-RoPE keys / values: E4M3 straight from the exact value when the K/V
    format is fp8 (the pipeline converts its float32 result once), else as ``prec``."""
    return round_fp8_e4m3(x) if kv == "fp8" else _rnd(x, prec)


def matmul_t(x: np.ndarray, w: np.ndarray, chunk: int = 16384) -> np.ndarray:
    """x @ w.T in float64 (w stored [out][in]); converted in row chunks of w to bound memory."""
    x = _f64(x)
    n_out = w.shape[0]
    out = np.empty(x.shape[:-1] + (n_out,), dtype=F64)
    for o in range(0, n_out, chunk):
        out[..., o:o + chunk] = x @ _f64(w[o:o + chunk]).T
    return out


# ---------------------------------------------------------------------------
# layer primitives
# ---------------------------------------------------------------------------
def rms_norm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _f64(g)


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary embedding, rotate-half convention: pair (i, i + hd/2) turns by pos * theta^(-2i/hd).

    x: [..., n, hd]; pos: [n] integer positions.
    """
    x = _f64(x)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = float(theta) ** (-(np.arange(half, dtype=F64) * 2.0) / hd)
    ang = np.asarray(pos, dtype=F64)[:, None] * inv_freq[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def attention(q, k, v, allowed: Optional[np.ndarray] = None, prec=None) -> np.ndarray:
    """softmax(q k^T / sqrt(hd)) v per query head; q [Hq][n][hd], k and v [Hkv][m][hd].

    Query head h reads kv head floor(h * Hkv / Hq).  ``allowed`` [n][m] masks keys.
    ``prec="bf16"``: the unnormalised probabilities exp(s - max s) that multiply the values are
    rounded to bfloat16 (a bf16 pipeline feeds them to its bf16 product with V); the normaliser
    sums them unrounded.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, n, hd = q.shape
    Hkv = k.shape[0]
    out = np.empty((Hq, n, v.shape[-1]), dtype=F64)
    for h in range(Hq):
        kv = (h * Hkv) // Hq
        s = q[h] @ k[kv].T / math.sqrt(hd)
        if allowed is not None:
            s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[h] = (_rnd(p, prec) @ v[kv]) / p.sum(axis=1, keepdims=True)
    return out


def silu(x) -> np.ndarray:
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def layer_forward(x, W: Dict[str, np.ndarray], li: int, dims, eps: float, theta: float, pos,
                  ctx_k=None, ctx_v=None, causal: bool = False, prec=None, kv=None):
    """One Qwen3-style block over the n rows ``x`` [n][d] of one sequence.

    ctx_k / ctx_v [Hkv][m][hd]: cached (post-RoPE) keys and values that every
    row sees in addition to the rows' own keys.  ``causal`` restricts the rows'
    own keys to positions <= the query's.  Returns (new x, k, v) where k and v
    [Hkv][n][hd] are this call's post-RoPE keys and values of the rows.

    ``prec="bf16"`` rounds to bfloat16 where a bf16 pipeline stores values: the
    normalised inputs of the projections, q / k / v, the attention probabilities that
    multiply the values, the attention output and the SwiGLU output (the residual stream
    stays exact).  Default: exact arithmetic.
    ``kv="fp8"``: keys and values are stored (and attended to) in FP8 E4M3.
    """
    p = "layers.%d." % li
    x = _f64(x)
    n = x.shape[0]
    Hq, Hkv, hd, F = dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn
    h1 = _rnd(rms_norm(x, W[p + "attn_norm"], eps), prec)
    qkv = matmul_t(h1, W[p + "wqkv"])
    q = qkv[:, : Hq * hd].reshape(n, Hq, hd).transpose(1, 0, 2)
    k = qkv[:, Hq * hd: (Hq + Hkv) * hd].reshape(n, Hkv, hd).transpose(1, 0, 2)
    v = _kv_round(qkv[:, (Hq + Hkv) * hd:].reshape(n, Hkv, hd).transpose(1, 0, 2), prec, kv)
    q = _rnd(rope(rms_norm(q, W[p + "q_norm"], eps), pos, theta), prec)
    k = _kv_round(rope(rms_norm(k, W[p + "k_norm"], eps), pos, theta), prec, kv)
    m = 0 if ctx_k is None else ctx_k.shape[1]
    keys = k if ctx_k is None else np.concatenate([_f64(ctx_k), k], axis=1)
    vals = v if ctx_v is None else np.concatenate([_f64(ctx_v), v], axis=1)
    allowed = None
    if causal:
        allowed = np.ones((n, m + n), dtype=bool)
        allowed[:, m:] = np.tril(np.ones((n, n), dtype=bool))
    a = _rnd(attention(q, keys, vals, allowed, prec).transpose(1, 0, 2).reshape(n, Hq * hd), prec)
    x = x + matmul_t(a, W[p + "wo"])
    h2 = _rnd(rms_norm(x, W[p + "ffn_norm"], eps), prec)
    gu = matmul_t(h2, W[p + "w_gate_up"])
    x = x + matmul_t(_rnd(silu(gu[:, :F]) * gu[:, F:], prec), W[p + "w_down"])
    return x, k, v


# ---------------------------------------------------------------------------
# the depth-aware prefix cache
# ---------------------------------------------------------------------------
def kv_slot(dims, k_max: int, layer: int, depth: int = 1) -> int:
    """Cache slot of (layer, loop depth): Prelude and Coda layers hold one set, Core layers k_max."""
    if layer < dims.n_pre:
        return layer
    if layer < dims.n_pre + dims.n_core:
        return dims.n_pre + (layer - dims.n_pre) * k_max + (depth - 1)
    return dims.n_pre + dims.n_core * k_max + (layer - dims.n_pre - dims.n_core)


def prefill_sequence(ids, W, dims, k_max: int, eps: float, theta: float, progress=None,
                     prec=None, depth: Optional[int] = None, state: bool = False, kv=None):
    """Depth-aware cache of one prefix: slot -> (K, V) [Hkv][P][hd] (causal prefix).
    ``progress`` (optional) is called with a short text after every layer call.

    ``depth`` (default k_max): build the Core only to this depth, the Coda set on the
    depth-``depth`` output (depth-on-demand prefill; every position's available depth is then
    ``depth``).  ``state``: also return the prefix's Core output at that depth, from which
    deepen_sequence continues.  ``kv`` as in layer_forward."""
    ids = np.asarray(ids)
    P = ids.shape[0]
    pos = np.arange(P)
    depth = k_max if depth is None else depth
    cache = {}
    x = _f64(W["embed"][ids])

    def run(li, slot):
        nonlocal x
        x, k, v = layer_forward(x, W, li, dims, eps, theta, pos, causal=True, prec=prec, kv=kv)
        cache[slot] = (k, v)
        if progress is not None:
            progress("prefill layer %d -> slot %d" % (li, slot))

    for li in range(dims.n_pre):
        run(li, kv_slot(dims, k_max, li))
    for dpt in range(1, depth + 1):
        for c in range(dims.n_core):
            run(dims.n_pre + c, kv_slot(dims, k_max, dims.n_pre + c, dpt))
    core_out = x
    for c in range(dims.n_coda):
        li = dims.n_pre + dims.n_core + c
        run(li, kv_slot(dims, k_max, li))
    return (cache, core_out) if state else cache


def deepen_sequence(cache, core_out, W, dims, k_max: int, eps: float, theta: float, depth_from: int,
                    depth_to: int, prec=None, kv=None):
    """Depth-on-demand: continue a prefix built to ``depth_from`` (its Core output ``core_out``)
    with the Core passes depth_from+1 .. depth_to, then rebuild the Coda set on the deeper output.
    Returns the deeper cache and Core output; equals the prefill built to ``depth_to`` directly."""
    P = core_out.shape[0]
    pos = np.arange(P)
    out = dict(cache)
    x = _f64(core_out)
    for dpt in range(depth_from + 1, depth_to + 1):
        for c in range(dims.n_core):
            li = dims.n_pre + c
            x, k, v = layer_forward(x, W, li, dims, eps, theta, pos, causal=True, prec=prec, kv=kv)
            out[kv_slot(dims, k_max, li, dpt)] = (k, v)
    core = x
    for c in range(dims.n_coda):
        li = dims.n_pre + dims.n_core + c
        x, k, v = layer_forward(x, W, li, dims, eps, theta, pos, causal=True, prec=prec, kv=kv)
        out[kv_slot(dims, k_max, li)] = (k, v)
    return out, core


def evict_depths(cache, avail, dims, k_max: int, keep: int, P: int):
    """Depth eviction: keep the Prelude and Coda sets and Core depths 1..``keep`` of a depth-aware
    cache of P positions, drop the deeper Core sets, and clip every available depth to ``keep``
    (``avail`` None: every position at k_max).  Returns the smaller cache and the clipped depths;
    a Core layer in loop s then reads position j at depth min(s, avail_j, keep)."""
    out = {}
    for li in range(dims.n_pre + dims.n_core + dims.n_coda):
        core = dims.n_pre <= li < dims.n_pre + dims.n_core
        for dpt in (range(1, keep + 1) if core else (1,)):
            slot = kv_slot(dims, k_max, li, dpt)
            if slot in cache:
                out[slot] = cache[slot]
    av = np.full(P, k_max, dtype=np.int64) if avail is None else np.asarray(avail, dtype=np.int64)
    return out, np.minimum(av, keep)


def context_for(cache, dims, k_max: int, layer: int, loop: int, avail):
    """Prefix K/V a block row reads at ``layer`` during loop ``loop`` (1-based).

    Core layers read prefix position j at depth min(loop, avail[j]); Prelude
    and Coda layers read their single set.
    """
    if dims.n_pre <= layer < dims.n_pre + dims.n_core:
        K0 = cache[kv_slot(dims, k_max, layer, 1)][0]
        P = K0.shape[1]
        depth = np.minimum(loop, np.asarray(avail, dtype=np.int64)) if avail is not None else np.full(P, loop)
        Ks = np.empty(K0.shape, dtype=F64)
        Vs = np.empty(K0.shape, dtype=F64)
        for dpt in np.unique(depth):
            sel = depth == dpt
            Kd, Vd = cache[kv_slot(dims, k_max, layer, int(dpt))]
            Ks[:, sel] = _f64(Kd[:, sel])
            Vs[:, sel] = _f64(Vd[:, sel])
        return Ks, Vs
    K, V = cache[kv_slot(dims, k_max, layer)]
    return _f64(K), _f64(V)


def extend_sequence(cache, avail, new_ids, W, dims, k_max: int, eps: float, theta: float, prec=None,
                    kv=None, keep: Optional[int] = None):
    """Appends positions (a finished block) to the depth-aware cache of one sequence.

    The new positions (ids ``new_ids``, positions P.. after the P cached ones) run through the
    Prelude once, the Core once per depth d = 1..k_max and the Coda once on the depth-k_max
    output, causally among themselves; cached position j is read as a step reads it (Core depth
    min(d, avail_j)).  Returns the longer cache (slot -> (K, V) [Hkv][P + n][hd]) and its
    available depths (the new positions at every depth).  ``keep`` < k_max: the cache holds
    depths 1..keep only (evict_depths); the new positions' deeper Core sets are dropped after
    use and their available depth is keep."""
    keep = k_max if keep is None else keep
    new_ids = np.asarray(new_ids)
    n = new_ids.shape[0]
    P = next(iter(cache.values()))[0].shape[1] if cache else 0
    pos = P + np.arange(n)
    x = _f64(W["embed"][new_ids])
    new = {}

    def run(li, depth):
        nonlocal x
        ck, cv = context_for(cache, dims, k_max, li, depth, avail) if cache else (None, None)
        x, k, v = layer_forward(x, W, li, dims, eps, theta, pos, ck, cv, causal=True, prec=prec, kv=kv)
        new[kv_slot(dims, k_max, li, depth)] = (k, v)

    for li in range(dims.n_pre):
        run(li, 1)
    for depth in range(1, k_max + 1):
        for c in range(dims.n_core):
            run(dims.n_pre + c, depth)
    for c in range(dims.n_coda):
        run(dims.n_pre + dims.n_core + c, 1)
    out = {}
    for li in range(dims.n_pre, dims.n_pre + dims.n_core):
        for dpt in range(keep + 1, k_max + 1):
            del new[kv_slot(dims, k_max, li, dpt)]
    for slot, (k, v) in new.items():
        if cache:
            out[slot] = (np.concatenate([_f64(cache[slot][0]), k], axis=1),
                         np.concatenate([_f64(cache[slot][1]), v], axis=1))
        else:
            out[slot] = (k, v)
    av0 = np.full(P, k_max, dtype=np.int64) if avail is None else np.asarray(avail, dtype=np.int64)
    return out, np.concatenate([av0, np.full(n, keep, dtype=np.int64)])


# ---------------------------------------------------------------------------
# the two heads
# ---------------------------------------------------------------------------
def readout(r, W_lm, boost_tok=None, boost_val=None, gumbel=None):
    """LMHead over readout rows r [n][d]: logits z = W_lm r (+ planted boost).

    Returns entropy H = -sum p ln p (nats), argmax token (lowest id on ties),
    log-sum-exp, and the gap between the two largest logits; with ``gumbel`` (noise [n][V])
    also the Gumbel-max draws of the rows and their top-2 gaps of z + g.
    """
    z = matmul_t(r, W_lm)
    n = z.shape[0]
    if boost_tok is not None:
        for i in range(n):
            if boost_tok[i] >= 0:
                z[i, boost_tok[i]] += float(boost_val[i])
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    S = e.sum(axis=1, keepdims=True)
    p = e / S
    logp = (z - m) - np.log(S)          # ln p, exact for every entry (no 0 * ln 0)
    H = -(p * logp).sum(axis=1)
    tok = np.argmax(z, axis=1).astype(np.int64)
    lse = (m + np.log(S))[:, 0]
    top2 = np.partition(z, z.shape[1] - 2, axis=1)[:, -2:]
    gap = np.abs(top2[:, 1] - top2[:, 0])
    if gumbel is not None:
        stok, sgap = gumbel_sample(z, gumbel)
        return H, tok, lse, gap, stok, sgap
    return H, tok, lse, gap


def exit_gate(r, w, b: float) -> np.ndarray:
    """Halting probability lambda = sigmoid(w . r + b) per row."""
    t = _f64(r) @ _f64(w) + float(b)
    return 1.0 / (1.0 + np.exp(-t))


# ---------------------------------------------------------------------------
# sampling commit: y ~ p by the Gumbel-max rule over counter-based uniforms
# ---------------------------------------------------------------------------
_MASK32 = 0xFFFFFFFF


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds (Salmon et al., SC'11): each round multiplies counter words 0
    and 2 by the two Philox constants into 64-bit products, the new words are (high of the
    second product) ^ c1 ^ k0, (low of the second), (high of the first) ^ c3 ^ k1, (low of the
    first); the key adds the two Weyl constants between rounds.  Vectorised over counters
    (uint64 arrays holding 32-bit words)."""
    c = [np.asarray(x, dtype=np.uint64) & np.uint64(_MASK32) for x in (c0, c1, c2, c3)]
    k0, k1 = np.uint64(k0 & _MASK32), np.uint64(k1 & _MASK32)
    m0, m1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
    w0, w1 = np.uint64(0x9E3779B9), np.uint64(0xBB67AE85)
    mask, sh = np.uint64(_MASK32), np.uint64(32)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + w0) & mask
            k1 = (k1 + w1) & mask
        p0 = c[0] * m0          # < 2^64: exact in uint64
        p1 = c[2] * m1
        c = [(p1 >> sh) ^ c[1] ^ k0, p1 & mask, (p0 >> sh) ^ c[3] ^ k1, p0 & mask]
    return c


def gumbel_noise(seed: int, step: int, b: int, i: int, s: int, V: int) -> np.ndarray:
    """Gumbel noise g_v, v < V, of block row i of sequence b at loop s: uniform
    u_v = (floor(x_v / 2^9) + 1/2) / 2^23 in (0, 1) from word v mod 4 of Philox4x32-10 at counter
    (v div 4, 64 b + i, s, step) and key (seed mod 2^32, seed div 2^32); g = -ln(-ln u)."""
    n = (V + 3) // 4
    g4 = np.arange(n, dtype=np.uint64)
    words = philox4x32_10(g4, np.full(n, 64 * b + i), np.full(n, s), np.full(n, step), seed & _MASK32,
                          (seed >> 32) & _MASK32)
    x = np.stack(words, axis=1).reshape(-1)[:V]            # word v mod 4 of group v div 4
    u = ((x >> np.uint64(9)).astype(F64) + 0.5) * 2.0 ** -23
    return -np.log(-np.log(u))


def gumbel_sample(z, g):
    """Draw y = argmax_v (z_v + g_v) per row (lowest v on ties): with g standard Gumbel noise,
    P(y = v) = softmax(z)_v.  Returns the draws and the gap between the two largest z + g."""
    y = _f64(z) + _f64(g)
    tok = np.argmax(y, axis=1).astype(np.int64)
    if y.shape[1] < 2:
        return tok, np.full(y.shape[0], np.inf)
    top2 = np.partition(y, y.shape[1] - 2, axis=1)[:, -2:]
    return tok, np.abs(top2[:, 1] - top2[:, 0])


# ---------------------------------------------------------------------------
# one denoising step of one sequence
# ---------------------------------------------------------------------------
def denoise_step_sequence(block_ids, cache, avail, W, dims, *, k_max: int, k_loops: int, eps: float,
                          theta: float, tau_ent: float, tau_halt: float, mask_id: int, exit_b: float,
                          boost_tok=None, boost_val=None, teacher: Optional[dict] = None,
                          record_hidden: bool = False, counter: Optional[list] = None, progress=None,
                          prec=None, sample: Optional[dict] = None, kv=None) -> dict:
    """One inner loop of Algorithm 1 of the summary page (one denoising step), for one sequence.

    ``cache``: slot -> (K, V) [Hkv][P][hd]; ``avail``: deepest cached Core depth
    per prefix position (None = k_max).  ``teacher`` (optional) replaces the
    decisions by given ones: {"commit_loop": [L], "tokens": [L], "stop_loop": int}.
    ``counter`` (optional list) receives one entry per layer call; ``progress`` (optional) is
    called with a short text after every layer call.  ``prec`` as in layer_forward (the
    readout rows feeding the LMHead are rounded too; the ExitGate reads them exactly).
    ``sample`` (optional) {"seed", "step", "seq"}: commit the Gumbel-max draw of each row
    (gumbel_noise with this sequence index) instead of its argmax.  ``kv="fp8"``: the rows' own keys
    and values are stored in FP8 E4M3 like the cache's.
    """
    block_ids = np.asarray(block_ids, dtype=np.int64)
    L = block_ids.shape[0]
    P = next(iter(cache.values()))[0].shape[1] if cache else 0
    pos = P + np.arange(L)

    def run_layer(x, li, loop):
        if counter is not None:
            counter.append(li)
        if cache:
            ck, cv = context_for(cache, dims, k_max, li, loop, avail)
        else:
            ck = cv = None
        y, _, _ = layer_forward(x, W, li, dims, eps, theta, pos, ck, cv, causal=False, prec=prec, kv=kv)
        if progress is not None:
            progress("step loop %d layer %d" % (loop, li))
        return y

    # start of the step: unresolved set, initial loop state, a = 0, C empty
    U = block_ids == mask_id
    C = np.zeros(L, dtype=bool)
    tokens = block_ids.copy()
    commit_loop = np.zeros(L, dtype=np.int64)
    if not U.any():   # nothing to denoise: no loop runs
        return dict(tokens=tokens, commit_loop=commit_loop, loops=0, records=[], forced=-1, forced_gap=float("nan"))
    a = np.zeros(L, dtype=F64)
    h = _f64(W["embed"][block_ids])
    for li in range(dims.n_pre):
        h = run_layer(h, li, 1)

    loops = []
    s_end = 0
    last = None
    for s in range(1, k_loops + 1):
        s_end = s
        # Core update, Coda readout
        y = h
        for c in range(dims.n_core):
            y = run_layer(y, dims.n_pre + c, s)
        h_tilde = y
        g = h_tilde
        for c in range(dims.n_coda):
            g = run_layer(g, dims.n_pre + dims.n_core + c, s)
        r = rms_norm(g, W["final_norm"], eps)
        rows = np.nonzero(U)[0]
        H = np.full(L, np.nan)
        tok = np.full(L, -1, dtype=np.int64)
        lse = np.full(L, np.nan)
        gap = np.full(L, np.nan)
        lam = np.full(L, np.nan)
        stok = np.full(L, -1, dtype=np.int64)
        sgap = np.full(L, np.nan)
        if rows.size:
            bt = None if boost_tok is None else np.asarray(boost_tok)[rows]
            bv = None if boost_val is None else np.asarray(boost_val)[rows]
            if sample is None:
                H[rows], tok[rows], lse[rows], gap[rows] = readout(_rnd(r[rows], prec), W["lm_head"], bt, bv)
            else:
                gn = np.stack([gumbel_noise(sample["seed"], sample["step"], sample["seq"], int(i), s,
                                            W["lm_head"].shape[0]) for i in rows])
                H[rows], tok[rows], lse[rows], gap[rows], stok[rows], sgap[rows] = readout(
                    _rnd(r[rows], prec), W["lm_head"], bt, bv, gumbel=gn)
            lam[rows] = exit_gate(r[rows], W["exit_w"], exit_b)
        ctok = tok if sample is None else stok   # the token a commit takes
        # cumulative halting for the positions unresolved at loop start
        a[rows] = a[rows] + (1.0 - a[rows]) * lam[rows]
        # entropy commit
        if teacher is None:
            newly = rows[H[rows] <= tau_ent]
        else:
            tcl = np.asarray(teacher["commit_loop"])
            newly = rows[tcl[rows] == s]
        for i in newly:
            tokens[i] = ctok[i] if teacher is None else int(teacher["tokens"][i])
            commit_loop[i] = s
        U[newly] = False
        C[newly] = True
        # Eq. 3: every row that is not unresolved re-enters as the embedding of its token
        h = h_tilde.copy()
        fixed = np.nonzero(~U)[0]
        if fixed.size:
            h[fixed] = _f64(W["embed"][tokens[fixed]])
        # stop test on the positions still unresolved
        n_u = int(U.sum())
        mean_a = float(a[U].mean()) if n_u else float("nan")
        if teacher is None:
            stop = n_u == 0 or mean_a >= tau_halt or s == k_loops
        else:
            stop = s == int(teacher["stop_loop"])
        rec = dict(loop=s, rows=rows, H=H, tok=tok, lse=lse, gap=gap, lam=lam, a=a.copy(),
                   committed=np.array(newly), mean_a=mean_a, n_unresolved=n_u, ctok=ctok)
        if sample is not None:
            rec["stok"] = stok
            rec["sgap"] = sgap
        if record_hidden:
            rec["h_tilde"] = h_tilde
            rec["h"] = h.copy()
            rec["r"] = r
        loops.append(rec)
        last = rec
        if stop:
            break

    # forced progress when the step committed nothing
    forced = -1
    forced_gap = float("nan")
    if not C.any() and U.any() and last is not None:
        cand = np.nonzero(U)[0]
        if teacher is None:
            Hc = last["H"][cand]
            forced = int(cand[np.argmin(Hc)])
            srt = np.sort(Hc)
            forced_gap = float(srt[1] - srt[0]) if srt.size > 1 else float("inf")
            tokens[forced] = last["ctok"][forced]
        else:
            tcl = np.asarray(teacher["commit_loop"])
            hits = cand[tcl[cand] == -s_end]
            if hits.size:
                forced = int(hits[0])
                tokens[forced] = int(teacher["tokens"][forced])
        if forced >= 0:
            commit_loop[forced] = -s_end
            U[forced] = False
    return dict(tokens=tokens, commit_loop=commit_loop, loops=s_end, records=loops, forced=forced,
                forced_gap=forced_gap)


def denoise_block_sequence(block_ids, cache, avail, W, dims, *, max_steps: Optional[int] = None,
                           sample: Optional[dict] = None, mask_id: int, **step_kw) -> dict:
    """Outer loop of Algorithm 1 over one sequence's block: denoising steps until no position is
    masked (or ``max_steps``), each starting from the block with the committed tokens written in.
    Every step commits at least one position (forced progress), so a block of L positions takes
    at most L steps.  ``sample`` {"seed", "step0"}: step t draws with counter word 3 = step0 + t - 1.
    ``step_kw``: the remaining arguments of denoise_step_sequence.  Returns the final ids, per
    position the step (1-based, 0 = not committed) and the loop of its commit, the number of
    steps and each step's result."""
    ids = np.asarray(block_ids, dtype=np.int64).copy()
    L = ids.shape[0]
    commit_step = np.zeros(L, dtype=np.int64)
    commit_loop = np.zeros(L, dtype=np.int64)
    results = []
    while (ids == mask_id).any() and (max_steps is None or len(results) < max_steps):
        t = len(results) + 1
        smp = None if sample is None else dict(seed=sample["seed"], step=sample["step0"] + t - 1,
                                               seq=sample["seq"])
        res = denoise_step_sequence(ids, cache, avail, W, dims, mask_id=mask_id, sample=smp, **step_kw)
        newly = res["commit_loop"] != 0
        commit_step[newly] = t
        commit_loop[newly] = res["commit_loop"][newly]
        ids = np.asarray(res["tokens"], dtype=np.int64).copy()
        results.append(res)
    return dict(tokens=ids, commit_step=commit_step, commit_loop=commit_loop, steps=len(results), results=results)


def readout_commit_group(r, W_lm, embed, exit_w, exit_b: float, tau_ent: float, tau_halt: float,
                         boost_tok=None, boost_val=None) -> dict:
    """The readout half of one loop for one group of rows that are all unresolved at loop 1
    with a = 0 and a loop cap of 1: heads, cumulative halt, commit, forced progress and the
    Eq. 3 embedding rows of the committed positions."""
    n = r.shape[0]
    H, tok, lse, gap = readout(r, W_lm, boost_tok, boost_val)
    lam = exit_gate(r, exit_w, exit_b)
    a = lam.copy()                           # a = 0 + (1 - 0) * lambda
    commit = H <= tau_ent
    # the stop test of the loop (Algorithm 1 (4)) averages a over the rows the entropy commits left
    # unresolved; forced progress (5) comes after it
    unresolved = ~commit
    mean_a = float(a[unresolved].mean()) if unresolved.any() else float("nan")
    commit_loop = np.where(commit, 1, 0).astype(np.int64)
    forced = -1
    if not commit.any() and n:
        forced = int(np.argmin(H))
        commit_loop[forced] = -1
    committed = commit_loop != 0
    emb = np.zeros((n, embed.shape[1]), dtype=F64)
    emb[committed] = _f64(embed[tok[committed]])
    return dict(H=H, tok=tok, lse=lse, gap=gap, lam=lam, a=a, commit_loop=commit_loop, forced=forced,
                mean_a=mean_a, embed_rows=emb)
