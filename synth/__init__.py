"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Nothing here scores, selects or compacts anything: this module only draws
random tensors (through the counter-based generator in ``gen.c``), rounds them
to bfloat16, and lays them out the way the library expects:

* ``Q``      bf16 bits, uint16 ``[Hq, n_q, D]``
* ``Kctx``   bf16 bits, uint16 ``[Hkv, n_ctx, D]`` (the context keys)
* ``Kself``  bf16 bits, uint16 ``[Hkv, n_q, D]`` (the repeated copy's own keys;
  repeat workloads only)
* ``V``      bf16 bits, uint16 ``[Hkv, n_ctx, D]``
* ``Vself``  bf16 bits, uint16 ``[Hkv, n_q, D]`` (the repeated copy's own
  values; repeat workloads with values only)
* ``WO``     bf16 bits, uint16 ``[d_model, Hkv * D]``: that random output
  projection (value-norm workloads only)
* ``vnorm``  fp32 ``[Hkv, n_ctx]``: the norm of a random output-projection
  block applied to each value row (the weight of the value-norm-normalised
  score); an *input* of the scoring call, synthesised here
* ``hnorm``  fp32 ``[n_q]``: residual-stream norms, log-normal

The recipes follow the workloads named in ``workloads.py``.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# stream ids: each tensor draws from its own counter-based stream
S_Q, S_QU, S_QB, S_K, S_KSELF, S_V, S_SINK, S_DUP, S_WO, S_HNORM = range(1, 11)
S_LSE, S_SCORES, S_TIES, S_PERM, S_VSELF = range(11, 16)


def build(verbose: bool = False) -> str:
    """Compile gen.c into libsynth.so with gcc (OpenMP)."""
    import subprocess

    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, d = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double
    vp = ctypes.c_void_p
    lib.synth_stream_key.argtypes = [u64, u64]
    lib.synth_stream_key.restype = u64
    lib.synth_u64.argtypes = [u64, u64, i64, vp]
    lib.synth_normal_f32.argtypes = [u64, u64, i64, d, d, vp]
    lib.synth_normal_f64.argtypes = [u64, u64, i64, d, d, vp]
    lib.synth_normal_bf16.argtypes = [u64, u64, i64, d, d, vp]
    lib.synth_f32_to_bf16.argtypes = [vp, i64, vp]
    _lib = lib
    return lib


def stream_key(seed: int, stream: int) -> int:
    return int(_load().synth_stream_key(seed & (2**64 - 1), stream))


def u64(seed: int, stream: int, count: int, first: int = 0) -> np.ndarray:
    out = np.empty(count, dtype=np.uint64)
    if count:
        _load().synth_u64(stream_key(seed, stream), first, count, out.ctypes.data)
    return out


def uniform(seed: int, stream: int, count: int, first: int = 0) -> np.ndarray:
    """Doubles in [0, 1) with 53 random bits."""
    return (u64(seed, stream, count, first) >> np.uint64(11)).astype(np.float64) * 2.0**-53


def normal_f64(seed, stream, shape, mean=0.0, std=1.0, first=0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float64)
    if n:
        _load().synth_normal_f64(stream_key(seed, stream), first, n, mean, std, out.ctypes.data)
    return out.reshape(shape)


def normal_f32(seed, stream, shape, mean=0.0, std=1.0, first=0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    if n:
        _load().synth_normal_f32(stream_key(seed, stream), first, n, mean, std, out.ctypes.data)
    return out.reshape(shape)


def normal_bf16(seed, stream, shape, mean=0.0, std=1.0, first=0) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    if n:
        _load().synth_normal_bf16(stream_key(seed, stream), first, n, mean, std, out.ctypes.data)
    return out.reshape(shape)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    if x.size:
        _load().synth_f32_to_bf16(x.ctypes.data, x.size, out.ctypes.data)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (a format conversion, not arithmetic)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def distinct_positions(seed, stream, count, lo, hi, first=0) -> np.ndarray:
    """`count` distinct integers drawn uniformly from [lo, hi), in draw order."""
    span = hi - lo
    if count > span:
        raise ValueError("more distinct positions than the range holds")
    seen, out, n = set(), [], first
    while len(out) < count:
        batch = u64(seed, stream, 4 * (count - len(out)) + 16, n)
        n += batch.size
        for x in batch:
            p = lo + int(x % np.uint64(span))
            if p not in seen:
                seen.add(p)
                out.append(p)
                if len(out) == count:
                    break
    return np.asarray(out, dtype=np.int64)


@dataclass(frozen=True)
class Recipe:
    """How to draw one attention layer's tensors (see module docstring)."""

    Hq: int
    Hkv: int
    D: int
    n_ctx: int
    n_q: int
    mask: str = "repeat"              # "repeat" or "causal"
    chunk: int = 0                    # repeat self-block length (0: whole n_q)
    scale: float = 0.0                # logit scale (0: 1/sqrt(D))
    q_prescale: float = 1.0           # multiply Q draws by this before rounding
    lowrank_rank: int = 0             # per-head low-rank component of Q
    lowrank_scale: float = 0.0        # per-entry std of that component
    sinks: int = 0                    # per KV head: rows of K scaled by sink_mult
    sink_mult: float = 4.0
    dup_frac: float = 0.0             # fraction of context rows copied from earlier rows
    value_norms: bool = False         # draw W_O, hnorm and derive vnorm
    d_hidden: int = 0                 # hidden size (0: Hq*D)
    wo_std: float = 0.02
    hnorm_mu: float = 3.0
    hnorm_sigma: float = 0.3
    with_values: bool = True

    @property
    def group(self) -> int:
        return self.Hq // self.Hkv

    @property
    def logit_scale(self) -> float:
        return float(np.float32(self.scale if self.scale else 1.0 / math.sqrt(self.D)))

    @property
    def self_chunk(self) -> int:
        return self.chunk if self.chunk else self.n_q


def draw(recipe: Recipe, seed: int) -> dict:
    """Draw every tensor of `recipe` with `seed`. Returns a dict of numpy arrays."""
    r = recipe
    out: dict = {"recipe": r, "seed": seed, "scale": r.logit_scale}

    # Q: N(0,1) (+ per-head rank-r component with per-entry std lowrank_scale)
    Q = np.empty((r.Hq, r.n_q, r.D), dtype=np.uint16)
    for g in range(r.Hq):
        z = normal_f64(seed, S_Q, (r.n_q, r.D), first=g * r.n_q * r.D)
        if r.lowrank_rank:
            U = normal_f64(seed, S_QU, (r.n_q, r.lowrank_rank), first=g * r.n_q * r.lowrank_rank)
            B = normal_f64(seed, S_QB, (r.lowrank_rank, r.D), first=g * r.lowrank_rank * r.D)
            z = z + (r.lowrank_scale / math.sqrt(r.lowrank_rank)) * (U @ B)
        qf = z.astype(np.float32)
        if r.q_prescale != 1.0:
            qf = qf * np.float32(r.q_prescale)
        Q[g] = f32_to_bf16(qf)
    out["Q"] = Q

    # context keys, with optional sinks
    if r.sinks:
        Kf = normal_f32(seed, S_K, (r.Hkv, r.n_ctx, r.D))
        sink_pos = np.zeros((r.Hkv, r.sinks), dtype=np.int64)
        for h in range(r.Hkv):
            sink_pos[h] = distinct_positions(seed, S_SINK, r.sinks, 0, r.n_ctx, first=h * 1_000_003)
            Kf[h, sink_pos[h]] *= np.float32(r.sink_mult)
        K = f32_to_bf16(Kf)
        out["sink_pos"] = sink_pos
        del Kf
    else:
        K = normal_bf16(seed, S_K, (r.Hkv, r.n_ctx, r.D))
    V = normal_bf16(seed, S_V, (r.Hkv, r.n_ctx, r.D)) if (r.with_values or r.value_norms) else None

    # duplicated context rows: positions p ascending, each copies an earlier row
    if r.dup_frac > 0 and r.n_ctx > 1:
        n_dup = int(r.dup_frac * r.n_ctx)
        pos = np.sort(distinct_positions(seed, S_DUP, n_dup, 1, r.n_ctx))
        src_u = u64(seed, S_DUP, n_dup, first=1 << 40)
        src = np.array([int(src_u[t] % np.uint64(p)) for t, p in enumerate(pos)], dtype=np.int64)
        for p, s in zip(pos, src):
            K[:, p] = K[:, s]
            if V is not None:
                V[:, p] = V[:, s]
        out["dup_pos"], out["dup_src"] = pos, src
    out["Kctx"] = K
    if V is not None:
        out["V"] = V

    if r.mask == "repeat":
        out["Kself"] = normal_bf16(seed, S_KSELF, (r.Hkv, r.n_q, r.D))
        if r.with_values:
            out["Vself"] = normal_bf16(seed, S_VSELF, (r.Hkv, r.n_q, r.D))

    if r.value_norms:
        dh = r.d_hidden if r.d_hidden else r.Hq * r.D
        WO = normal_bf16(seed, S_WO, (dh, r.Hkv * r.D), std=r.wo_std)
        Wf = bf16_to_f32(WO).astype(np.float64)
        vnorm = np.empty((r.Hkv, r.n_ctx), dtype=np.float32)
        for h in range(r.Hkv):
            Wh = Wf[:, h * r.D:(h + 1) * r.D]
            gram = Wh.T @ Wh                                   # [D, D]
            v = bf16_to_f32(V[h]).astype(np.float64)           # [n_ctx, D]
            sq = np.einsum("nd,nd->n", v @ gram, v)
            vnorm[h] = np.sqrt(np.maximum(sq, 0.0)).astype(np.float32)
        out["vnorm"] = vnorm
        out["WO"] = WO
        out["hnorm"] = np.exp(normal_f64(seed, S_HNORM, (r.n_q,), r.hnorm_mu, r.hnorm_sigma)).astype(np.float32)
    return out


def lse_values(seed: int, Hq: int, n_q: int, lo: float, hi: float) -> np.ndarray:
    """Uniform fp32 values in [lo, hi), shape [Hq, n_q]: a stand-in row normaliser
    that does not come from any attention computation."""
    return (lo + (hi - lo) * uniform(seed, S_LSE, Hq * n_q)).astype(np.float32).reshape(Hq, n_q)


def evict_scores(seed: int, Hkv: int, n: int, *, tie_frac: float = 0.05,
                 zero_frac: float = 0.0, mu: float = -6.0, sigma: float = 2.0) -> np.ndarray:
    """Log-normal fp32 scores [Hkv, n] with exact ties (a fraction of entries
    copied from other entries) and an optional fraction of exact zeros."""
    s = np.exp(normal_f64(seed, S_SCORES, (Hkv, n), mu, sigma)).astype(np.float32)
    if n > 1 and tie_frac > 0:
        m = int(tie_frac * n)
        u = u64(seed, S_TIES, 2 * Hkv * m).reshape(Hkv, 2 * m) % np.uint64(n)
        for h in range(Hkv):
            s[h, u[h, :m].astype(np.int64)] = s[h, u[h, m:].astype(np.int64)]
    if zero_frac > 0:
        m = int(zero_frac * n)
        u = u64(seed, S_PERM, Hkv * m).reshape(Hkv, m) % np.uint64(n)
        for h in range(Hkv):
            s[h, u[h].astype(np.int64)] = 0.0
    return s
