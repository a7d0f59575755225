"""Python binding of libkvscore (KV-cache importance scoring and eviction on
MI355X / gfx950).

Argument marshalling only: every step runs in the library's HIP kernels.
Torch supplies device memory and the current stream. The functions mirror
the C ABI in ``include/kvscore.h``:

* :func:`lse`          -> ``kvscore_lse``
* :func:`attention`    -> ``kvscore_attention``
* :func:`value_norms`  -> ``kvscore_vnorm``
* :func:`decode`       -> ``kvscore_decode`` (+ ``kvscore_decode_workspace_bytes``)
* :func:`max_scores`   -> ``kvscore_max``
* :func:`future_mass`  -> ``kvscore_futuremass``
* :func:`evict`        -> ``kv_evict`` (+ ``kv_evict_workspace_bytes``)
* :func:`evict_noalloc` -> ``kv_evict_noalloc`` (no workspace argument; allocates nothing)
* :class:`StreamCache` -> ``kv_stream_append`` (threshold pruning as tokens arrive)

Tensors: bf16 ``[heads, tokens, head_dim]`` with a contiguous last dimension
(any head/token strides that keep rows 16-byte aligned), fp32 normalisers and
scores. The library allocates nothing; outputs are allocated here with torch
when not given.
"""
from __future__ import annotations

import ctypes
import os

from . import accounting  # noqa: F401  (host-side, no GPU needed)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvscore.so")

KVS_OK, KVS_EINVAL, KVS_EUNSUPPORTED, KVS_ECAPACITY, KVS_EWORKSPACE, KVS_EHIP, KVS_ENODEV = range(7)
MASK_REPEAT, MASK_CAUSAL = 0, 1

EXPORTED_SYMBOLS = (
    "kvscore_lse", "kvscore_attention", "kvscore_vnorm", "kvscore_decode_workspace_bytes", "kvscore_decode",
    "kvscore_max", "kvscore_futuremass", "kv_evict_workspace_bytes", "kv_evict", "kv_evict_noalloc",
    "kv_stream_append",
    "kvs_strerror", "kvs_last_error", "kvs_version",
)


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("n_qheads", ctypes.c_int32), ("n_kvheads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("mask", ctypes.c_int32),
        ("n_ctx", ctypes.c_int64), ("n_q", ctypes.c_int64), ("chunk", ctypes.c_int64),
        ("q_head_stride", ctypes.c_int64), ("q_tok_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64), ("k_tok_stride", ctypes.c_int64),
        ("ks_head_stride", ctypes.c_int64), ("ks_tok_stride", ctypes.c_int64),
        ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


class EvictDesc(ctypes.Structure):
    _fields_ = [
        ("n_kvheads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_tok", ctypes.c_int64), ("k", ctypes.c_int64),
        ("tau", ctypes.c_float), ("scope", ctypes.c_int32),
        ("window", ctypes.c_int64), ("capacity", ctypes.c_int64),
        ("kv_head_stride", ctypes.c_int64), ("kv_tok_stride", ctypes.c_int64),
        ("score_head_stride", ctypes.c_int64),
    ]


class VnormDesc(ctypes.Structure):
    _fields_ = [
        ("n_kvheads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_tok", ctypes.c_int64),
        ("d_model", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("v_head_stride", ctypes.c_int64), ("v_tok_stride", ctypes.c_int64),
        ("wo_row_stride", ctypes.c_int64),
    ]


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("n_qheads", ctypes.c_int32), ("n_kvheads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("n_q", ctypes.c_int32),
        ("q_head_stride", ctypes.c_int64), ("q_tok_stride", ctypes.c_int64),
        ("capacity", ctypes.c_int64),
        ("scale", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("head_stride_rows", ctypes.c_int64),
    ]


class StreamDesc(ctypes.Structure):
    _fields_ = [
        ("n_kvheads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("n_seen", ctypes.c_int64), ("n_new", ctypes.c_int64), ("window", ctypes.c_int64),
        ("tau", ctypes.c_float), ("reserved", ctypes.c_int32),
        ("capacity", ctypes.c_int64),
        ("new_head_stride", ctypes.c_int64), ("new_tok_stride", ctypes.c_int64),
        ("score_head_stride", ctypes.c_int64),
    ]


class KvsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvscore.so (built in-tree by ``build.build()``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_eviction_lse_amd.build` "
                          "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, c = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int
    pA, pE = ctypes.POINTER(AttnDesc), ctypes.POINTER(EvictDesc)
    L.kvscore_lse.argtypes = [pA, vp, vp, vp, vp, vp]
    L.kvscore_attention.argtypes = [pA, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kvscore_vnorm.argtypes = [ctypes.POINTER(VnormDesc), vp, vp, vp, vp]
    pD = ctypes.POINTER(DecodeDesc)
    L.kvscore_decode_workspace_bytes.argtypes = [pD]
    L.kvscore_decode_workspace_bytes.restype = ctypes.c_size_t
    L.kvscore_decode.argtypes = [pD, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.kvscore_max.argtypes = [pA, vp, vp, vp, vp, vp, vp, c, vp]
    L.kvscore_futuremass.argtypes = [pA, vp, vp, vp, i64, vp, vp, vp, vp]
    L.kv_evict_workspace_bytes.argtypes = [pE]
    L.kv_evict_workspace_bytes.restype = ctypes.c_size_t
    L.kv_evict.argtypes = [pE, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.kv_evict_noalloc.argtypes = [pE, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kv_stream_append.argtypes = [ctypes.POINTER(StreamDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.kvs_strerror.argtypes = [i32]
    L.kvs_strerror.restype = ctypes.c_char_p
    L.kvs_last_error.argtypes = []
    L.kvs_last_error.restype = ctypes.c_char_p
    L.kvs_version.restype = c
    for name in ("kvscore_lse", "kvscore_attention", "kvscore_vnorm", "kvscore_decode", "kvscore_max", "kvscore_futuremass", "kv_evict",
                 "kv_evict_noalloc", "kv_stream_append"):
        getattr(L, name).restype = c
    _lib = L
    return L


def check(status: int) -> None:
    if status != KVS_OK:
        L = lib()
        raise KvsError(status, f"{L.kvs_strerror(status).decode()}: {L.kvs_last_error().decode()}")


# ---------------------------------------------------------------- helpers

def _torch():
    import torch

    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _bf16(name, t, ndim=3):
    """dtype and layout of a bf16 operand (the device is checked by _on_gpu,
    after the shape checks, so that those also run on a host without a GPU)."""
    torch = _torch()
    if t is None or not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
    if t.dim() != ndim or t.stride(-1) != 1:
        raise ValueError(f"{name} must be [heads, tokens, head_dim] with a contiguous last dimension")
    return t


def _f32(name, t, shape):
    torch = _torch()
    if t is None:
        return None
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")
    return t


def _on_gpu(**tensors):
    """Every given tensor (None skipped) must be on the GPU."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")


def _check_kself(K, Kself, n_q):
    """REPEAT self keys: [Hkv, n_q, D] with K's head count and head_dim."""
    if tuple(Kself.shape) != (K.shape[0], n_q, K.shape[2]):
        raise ValueError(f"Kself must be [Hkv, n_q, D] = {(K.shape[0], n_q, K.shape[2])}, got {tuple(Kself.shape)}")


def attn_desc(Q, K, Kself, scale, mask, chunk) -> AttnDesc:
    Hq, n_q, D = Q.shape
    Hkv, n_ctx, Dk = K.shape
    if Dk != D:
        raise ValueError("Q and K head_dim differ")
    if Kself is not None:
        _check_kself(K, Kself, n_q)
    d = AttnDesc()
    d.n_qheads, d.n_kvheads, d.head_dim = Hq, Hkv, D
    d.mask = MASK_REPEAT if mask == "repeat" else MASK_CAUSAL
    d.n_ctx, d.n_q = n_ctx, n_q
    d.chunk = chunk if chunk else max(n_q, 1)
    d.q_head_stride, d.q_tok_stride = Q.stride(0), Q.stride(1)
    d.k_head_stride, d.k_tok_stride = K.stride(0), K.stride(1)
    if Kself is not None:
        d.ks_head_stride, d.ks_tok_stride = Kself.stride(0), Kself.stride(1)
    d.scale = float(scale)
    d.reserved = 0
    return d


# ---------------------------------------------------------------- entry points

def lse(Q, K, Kself=None, *, scale: float, mask: str = "repeat", chunk: int = 0, out=None, stream=None):
    """Per-query log-sum-exp [Hq, n_q] fp32 (``kvscore_lse``)."""
    torch = _torch()
    _bf16("Q", Q), _bf16("K", K)
    if mask == "repeat":
        _bf16("Kself", Kself)
    d = attn_desc(Q, K, Kself, scale, mask, chunk)
    if out is None:
        out = torch.empty((d.n_qheads, d.n_q), dtype=torch.float32, device=Q.device)
    _f32("out", out, (d.n_qheads, d.n_q))
    _on_gpu(Q=Q, K=K, Kself=Kself, out=out)
    check(lib().kvscore_lse(ctypes.byref(d), _ptr(Q), _ptr(K), _ptr(Kself), _ptr(out), _stream(stream)))
    return out


def attention(Q, K, V, Kself=None, Vself=None, *, scale: float, mask: str = "repeat", chunk: int = 0,
              out=None, lse_out=None, stream=None):
    """Attention output O (bf16, Q's shape and strides) and LSE [Hq, n_q] fp32
    (``kvscore_attention``). V has K's shape and strides, Vself Kself's."""
    torch = _torch()
    _bf16("Q", Q), _bf16("K", K), _bf16("V", V)
    if tuple(V.shape) != tuple(K.shape) or V.stride() != K.stride():
        raise ValueError("V must have K's shape and strides")
    if mask == "repeat":
        _bf16("Kself", Kself), _bf16("Vself", Vself)
        if tuple(Vself.shape) != tuple(Kself.shape) or Vself.stride() != Kself.stride():
            raise ValueError("Vself must have Kself's shape and strides")
    d = attn_desc(Q, K, Kself, scale, mask, chunk)
    if out is None:
        out = torch.empty_like(Q)
    _bf16("out", out)
    if tuple(out.shape) != tuple(Q.shape) or out.stride() != Q.stride():
        raise ValueError("out must have Q's shape and strides")
    if lse_out is None:
        lse_out = torch.empty((d.n_qheads, d.n_q), dtype=torch.float32, device=Q.device)
    _f32("lse_out", lse_out, (d.n_qheads, d.n_q))
    _on_gpu(Q=Q, K=K, V=V, Kself=Kself, Vself=Vself, out=out, lse_out=lse_out)
    check(lib().kvscore_attention(ctypes.byref(d), _ptr(Q), _ptr(K), _ptr(Kself), _ptr(V), _ptr(Vself),
                                  _ptr(out), _ptr(lse_out), _stream(stream)))
    return out, lse_out


def value_norms(V, W_O, *, out=None, stream=None):
    """||W_O v_i|| per KV head and key, fp32 [Hkv, n] (``kvscore_vnorm``).
    V bf16 [Hkv, n, D]; W_O bf16 [d_model, Hkv * D] with a contiguous last dimension."""
    torch = _torch()
    _bf16("V", V)
    if W_O.dtype != torch.bfloat16 or W_O.dim() != 2 or W_O.stride(-1) != 1:
        raise ValueError("W_O must be a bfloat16 matrix [d_model, Hkv * D] with a contiguous last dimension")
    Hkv, n, D = V.shape
    if W_O.shape[1] != Hkv * D:
        raise ValueError("W_O must have Hkv * D columns")
    d = VnormDesc()
    d.n_kvheads, d.head_dim, d.n_tok, d.d_model, d.reserved = Hkv, D, n, W_O.shape[0], 0
    d.v_head_stride, d.v_tok_stride, d.wo_row_stride = V.stride(0), V.stride(1), W_O.stride(0)
    if out is None:
        out = torch.empty((Hkv, n), dtype=torch.float32, device=V.device)
    _f32("out", out, (Hkv, n))
    _on_gpu(V=V, W_O=W_O, out=out)
    check(lib().kvscore_vnorm(ctypes.byref(d), _ptr(V), _ptr(W_O), _ptr(out), _stream(stream)))
    return out


def decode_desc(Q, K_cache, n_kvheads, scale, head_stride_rows: int = 0) -> DecodeDesc:
    Hq, n_q, D = Q.shape
    d = DecodeDesc()
    d.n_qheads, d.n_kvheads, d.head_dim, d.n_q = Hq, n_kvheads, D, n_q
    d.q_head_stride, d.q_tok_stride = Q.stride(0), Q.stride(1)
    d.capacity = K_cache.shape[0]
    d.scale, d.reserved = float(scale), 0
    d.head_stride_rows = int(head_stride_rows)
    return d


def decode_workspace_bytes(d: DecodeDesc) -> int:
    return int(lib().kvscore_decode_workspace_bytes(ctypes.byref(d)))


def decode(Q, K_cache, V_cache, head_offsets, *, scale: float, workspace=None, out=None, lse_out=None,
           head_stride_rows: int = 0, stream=None):
    """Decode attention of Q [Hq, n_q, D] over the compacted per-head cache
    (``kvscore_decode``): K_cache/V_cache [capacity, D] bf16 rows and the
    device int64 head_offsets [Hkv+1] that kv_evict wrote; or, with
    ``head_stride_rows`` = S > 0, per-head regions of S rows and live row
    counts head_offsets [Hkv] (a StreamCache's layout). Returns (O, lse)."""
    torch = _torch()
    _bf16("Q", Q)
    for name, t in (("K_cache", K_cache), ("V_cache", V_cache)):
        if t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 matrix [capacity, D]")
    if K_cache.shape != V_cache.shape or K_cache.shape[1] != Q.shape[2]:
        raise ValueError("K_cache and V_cache must be [capacity, D] with Q's D")
    if head_offsets.dtype != torch.int64 or head_offsets.dim() != 1:
        raise ValueError("head_offsets must be an int64 vector ([Hkv + 1], or [Hkv] with head_stride_rows)")
    n_kv = head_offsets.numel() - (0 if head_stride_rows else 1)
    d = decode_desc(Q, K_cache, n_kv, scale, head_stride_rows)
    need = decode_workspace_bytes(d)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=Q.device)
    if out is None:
        out = torch.empty_like(Q)
    _bf16("out", out)
    if tuple(out.shape) != tuple(Q.shape) or out.stride() != Q.stride():
        raise ValueError("out must have Q's shape and strides")
    if lse_out is None:
        lse_out = torch.empty((d.n_qheads, d.n_q), dtype=torch.float32, device=Q.device)
    _f32("lse_out", lse_out, (d.n_qheads, d.n_q))
    _on_gpu(Q=Q, K_cache=K_cache, V_cache=V_cache, head_offsets=head_offsets, workspace=workspace, out=out,
            lse_out=lse_out)
    check(lib().kvscore_decode(ctypes.byref(d), _ptr(Q), _ptr(K_cache), _ptr(V_cache), _ptr(head_offsets),
                               _ptr(out), _ptr(lse_out), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse_out


def max_scores(Q, K, lse_vals, *, scale: float, vnorm=None, hnorm=None, out=None, accumulate: bool = False,
               stream=None):
    """KVzip / KVzip+ max score per context key [Hkv, n_ctx] fp32 (``kvscore_max``)."""
    torch = _torch()
    _bf16("Q", Q), _bf16("K", K)
    d = attn_desc(Q, K, None, scale, "repeat", 0)
    _f32("lse", lse_vals, (d.n_qheads, d.n_q))
    _f32("vnorm", vnorm, (d.n_kvheads, d.n_ctx))
    _f32("hnorm", hnorm, (d.n_q,))
    if out is None:
        if accumulate:
            raise ValueError("accumulate needs an existing out tensor")
        out = torch.empty((d.n_kvheads, d.n_ctx), dtype=torch.float32, device=Q.device)
    _f32("out", out, (d.n_kvheads, d.n_ctx))
    _on_gpu(Q=Q, K=K, lse=lse_vals, vnorm=vnorm, hnorm=hnorm, out=out)
    check(lib().kvscore_max(ctypes.byref(d), _ptr(Q), _ptr(K), _ptr(lse_vals), _ptr(vnorm), _ptr(hnorm),
                            _ptr(out), 1 if accumulate else 0, _stream(stream)))
    return out


def future_mass(Q, K, lse_vals, *, scale: float, window: int, vnorm=None, hnorm=None, out=None, stream=None):
    """KVpop future-attention target per key [Hkv, T] fp32 (``kvscore_futuremass``)."""
    torch = _torch()
    _bf16("Q", Q), _bf16("K", K)
    d = attn_desc(Q, K, None, scale, "causal", 0)
    _f32("lse", lse_vals, (d.n_qheads, d.n_q))
    _f32("vnorm", vnorm, (d.n_kvheads, d.n_ctx))
    _f32("hnorm", hnorm, (d.n_q,))
    if out is None:
        out = torch.empty((d.n_kvheads, d.n_ctx), dtype=torch.float32, device=Q.device)
    _f32("out", out, (d.n_kvheads, d.n_ctx))
    _on_gpu(Q=Q, K=K, lse=lse_vals, vnorm=vnorm, hnorm=hnorm, out=out)
    check(lib().kvscore_futuremass(ctypes.byref(d), _ptr(Q), _ptr(K), _ptr(lse_vals), int(window), _ptr(vnorm),
                                   _ptr(hnorm), _ptr(out), _stream(stream)))
    return out


SCOPE_HEAD, SCOPE_LAYER = 0, 1


def evict_desc(scores, K, *, window: int, k=None, tau=None, capacity=None, scope: str = "head") -> EvictDesc:
    if (k is None) == (tau is None):
        raise ValueError("give exactly one of k, tau")
    if scope not in ("head", "layer"):
        raise ValueError("scope must be 'head' or 'layer'")
    Hkv, n, D = K.shape
    e = EvictDesc()
    e.n_kvheads, e.head_dim, e.n_tok = Hkv, D, n
    e.k = int(k) if k is not None else -1
    e.tau = float(tau) if tau is not None else 0.0
    e.scope = SCOPE_LAYER if scope == "layer" else SCOPE_HEAD
    e.window = int(window)
    w = min(int(window), n)
    if k is None:
        need = Hkv * n
    elif scope == "layer":
        need = Hkv * w + min(int(k), Hkv * (n - w))
    else:
        need = Hkv * (w + min(int(k), n - w))
    e.capacity = need if capacity is None else int(capacity)
    e.kv_head_stride, e.kv_tok_stride = K.stride(0), K.stride(1)
    e.score_head_stride = scores.stride(0)
    return e


def evict_workspace_bytes(desc: EvictDesc) -> int:
    return int(lib().kv_evict_workspace_bytes(ctypes.byref(desc)))


def torch_empty_bytes(n: int, device):
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def _evict_prepare(scores, K, V, window, k, tau, capacity, outputs, scope):
    """Shared argument checks of evict / evict_noalloc; returns the descriptor
    and the four output tensors (allocated here when not given)."""
    torch = _torch()
    _bf16("K", K), _bf16("V", V)
    if K.shape != V.shape or K.stride() != V.stride():
        raise ValueError("K and V must have the same shape and strides")
    Hkv, n, D = K.shape
    if scores.dtype != torch.float32 or scores.dim() != 2 or (scores.numel() and scores.stride(1) != 1):
        raise ValueError("scores must be float32 [Hkv, n] with contiguous rows")
    if tuple(scores.shape) != (Hkv, n):
        raise ValueError(f"scores must be [Hkv, n] = {(Hkv, n)}, got {tuple(scores.shape)}")
    e = evict_desc(scores, K, window=window, k=k, tau=tau, capacity=capacity, scope=scope)
    dev = K.device
    if outputs is None:
        kept = torch.empty(max(e.capacity, 1), dtype=torch.int32, device=dev)
        offs = torch.empty(e.n_kvheads + 1, dtype=torch.int64, device=dev)
        Ko = torch.empty((max(e.capacity, 1), e.head_dim), dtype=torch.bfloat16, device=dev)
        Vo = torch.empty((max(e.capacity, 1), e.head_dim), dtype=torch.bfloat16, device=dev)
    else:
        kept, offs, Ko, Vo = outputs
        if kept.dtype != torch.int32 or kept.dim() != 1 or not kept.is_contiguous() or kept.numel() < e.capacity:
            raise ValueError(f"kept_idx must be a contiguous int32 vector of at least {e.capacity} entries")
        if offs.dtype != torch.int64 or offs.dim() != 1 or not offs.is_contiguous() or offs.numel() < Hkv + 1:
            raise ValueError(f"head_offsets must be a contiguous int64 vector of at least {Hkv + 1} entries")
        for name, t in (("K_out", Ko), ("V_out", Vo)):
            if (t.dtype != torch.bfloat16 or t.dim() != 2 or not t.is_contiguous() or t.shape[1] != D
                    or t.shape[0] < e.capacity):
                raise ValueError(f"{name} must be a contiguous bfloat16 [>= {e.capacity}, {D}] matrix")
    _on_gpu(kept_idx=kept, head_offsets=offs, K_out=Ko, V_out=Vo)
    return e, (kept, offs, Ko, Vo)


def evict(scores, K, V, *, window: int, k=None, tau=None, capacity=None, workspace=None, outputs=None,
          scope: str = "head", stream=None):
    """Keep the window plus top-k / tau-passing keys per KV head and compact K, V
    (``kv_evict``); ``scope="layer"`` makes k one budget for all heads together.
    Returns (kept_idx int32 [capacity], head_offsets int64 [Hkv+1],
    K_out, V_out bf16 [capacity, D]); rows past head_offsets[-1] are unused."""
    e, (kept, offs, Ko, Vo) = _evict_prepare(scores, K, V, window, k, tau, capacity, outputs, scope)
    nbytes = evict_workspace_bytes(e)
    if workspace is None:
        workspace = torch_empty_bytes(max(nbytes, 256), K.device)
    if workspace.dtype != _torch().uint8 or workspace.dim() != 1:
        raise ValueError("workspace must be a uint8 vector")
    _on_gpu(scores=scores, K=K, V=V, workspace=workspace)
    check(lib().kv_evict(ctypes.byref(e), _ptr(scores), _ptr(K), _ptr(V), _ptr(kept), _ptr(offs), _ptr(Ko),
                         _ptr(Vo), _ptr(workspace), workspace.numel(), _stream(stream)))
    return kept, offs, Ko, Vo


# kv_evict_noalloc's fixed scratch (KVS_EVICT_NOALLOC_MAX_WORKSPACE in the header)
EVICT_NOALLOC_MAX_WORKSPACE = 4 << 20


def evict_noalloc(scores, K, V, *, window: int, outputs, k=None, tau=None, capacity=None, scope: str = "head",
                  stream=None):
    """``kv_evict_noalloc``: :func:`evict` without a workspace argument, for
    callers that cannot allocate device memory. ``outputs`` (kept_idx,
    head_offsets, K_out, V_out) must be given: nothing is allocated here or
    in the library. Calls that can overlap in time on one GPU share the
    library's scratch and race."""
    if outputs is None:
        raise ValueError("evict_noalloc allocates nothing: pass outputs=(kept_idx, head_offsets, K_out, V_out)")
    e, (kept, offs, Ko, Vo) = _evict_prepare(scores, K, V, window, k, tau, capacity, outputs, scope)
    _on_gpu(scores=scores, K=K, V=V)
    check(lib().kv_evict_noalloc(ctypes.byref(e), _ptr(scores), _ptr(K), _ptr(V), _ptr(kept), _ptr(offs), _ptr(Ko),
                                 _ptr(Vo), _stream(stream)))
    return kept, offs, Ko, Vo


class StreamCache:
    """One layer's cache under threshold pruning as tokens arrive
    (``kv_stream_append``): per KV head a region of ``capacity`` rows, the
    window ring in rows [0, window) (position p in row p mod window), then
    the kept tokens that left the window, ascending. ``head_len`` [Hkv]
    (device) holds each head's live rows, rows [0, head_len[h]) of its
    region; ``decode`` attends to exactly those. The library allocates
    nothing: the tensors are allocated here with torch."""

    def __init__(self, n_kvheads: int, head_dim: int, capacity: int, *, window: int, tau: float, device="cuda"):
        torch = _torch()
        self.n_kvheads, self.head_dim, self.capacity = int(n_kvheads), int(head_dim), int(capacity)
        self.window, self.tau, self.n_seen = int(window), float(tau), 0
        self.K = torch.zeros((self.n_kvheads, self.capacity, self.head_dim), dtype=torch.bfloat16, device=device)
        self.V = torch.zeros_like(self.K)
        self.pos = torch.full((self.n_kvheads, self.capacity), -1, dtype=torch.int32, device=device)
        self.win_scores = torch.zeros((self.n_kvheads, max(self.window, 1)), dtype=torch.float32, device=device)
        self.head_len = torch.zeros(self.n_kvheads, dtype=torch.int64, device=device)

    def desc(self, new_scores, K_new) -> StreamDesc:
        d = StreamDesc()
        d.n_kvheads, d.head_dim = self.n_kvheads, self.head_dim
        d.n_seen, d.n_new, d.window = self.n_seen, K_new.shape[1], self.window
        d.tau, d.reserved = self.tau, 0
        d.capacity = self.capacity
        d.new_head_stride, d.new_tok_stride = K_new.stride(0), K_new.stride(1)
        d.score_head_stride = new_scores.stride(0)
        return d

    def append(self, new_scores, K_new, V_new, stream=None) -> None:
        """Append n_new tokens per head: new_scores fp32 [Hkv, n_new] (contiguous
        rows), K_new / V_new bf16 [Hkv, n_new, D] with equal strides."""
        torch = _torch()
        _bf16("K_new", K_new), _bf16("V_new", V_new)
        if K_new.shape != V_new.shape or K_new.stride() != V_new.stride():
            raise ValueError("K_new and V_new must have the same shape and strides")
        if tuple(K_new.shape[::2]) != (self.n_kvheads, self.head_dim):
            raise ValueError("K_new must be [n_kvheads, n_new, head_dim]")
        if new_scores.dtype != torch.float32 or tuple(new_scores.shape) != tuple(K_new.shape[:2]) \
                or (new_scores.numel() and new_scores.stride(1) != 1):
            raise ValueError("new_scores must be float32 [n_kvheads, n_new] with contiguous rows")
        d = self.desc(new_scores, K_new)
        _on_gpu(new_scores=new_scores, K_new=K_new, V_new=V_new)
        check(lib().kv_stream_append(ctypes.byref(d), _ptr(new_scores), _ptr(K_new), _ptr(V_new), _ptr(self.K),
                                     _ptr(self.V), _ptr(self.pos), _ptr(self.win_scores), _ptr(self.head_len),
                                     _stream(stream)))
        self.n_seen += int(K_new.shape[1])

    def decode(self, Q, *, scale: float, workspace=None, out=None, lse_out=None, stream=None):
        """Decode attention of Q [Hq, n_q, D] over every head's live rows."""
        flat = (self.n_kvheads * self.capacity, self.head_dim)
        return decode(Q, self.K.view(flat), self.V.view(flat), self.head_len, scale=scale, workspace=workspace,
                      out=out, lse_out=lse_out, head_stride_rows=self.capacity, stream=stream)
