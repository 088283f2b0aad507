"""MI355X (gfx950) sliding-window / global attention with per-head sinks.

Thin ctypes binding over ``libswa_attn.so`` (the HIP kernels behind the C ABI
declared in ``include/swa_attn.h``).  The functions carry the C names:

    swa_attn_prefill(q, k, v, sinks, window, q_offset=0, sm_scale=None, out=None)
    swa_attn_verify_workspace_bytes(...)
    swa_attn_verify(q, k_new, v_new, k_cache, v_cache, cache_len, sinks, window, ring, ...)
    swa_attn_verify_noalloc(q, k_new, v_new, k_cache, v_cache, cache_len, sinks, window, ring, ...)
    kv_ring_append(k_cache, v_cache, k_new, v_new, cache_len, n_append, ring)
    swa_mtp_accept_workspace_bytes(B, q_len, vocab)
    swa_mtp_greedy_accept(logits, draft, ...) -> (target, n_append)
    swa_cache_advance(cache_len, n_append)
    swa_rope_apply(x, rot_dim, base, pos0=None, pos_offset=0)
    swa_attn_prefill_rope(q, k, v, sinks, window, rot_dim, rope_base, q_offset=0, ...)
    swa_attn_prefill_lse(q, k, v, sinks, window, q_offset=0, ...) -> (o, lse)
    swa_attn_backward(q, k, v, sinks, o, lse, dout, window, ...) -> (dq, dk, dv, dsink)

They only check and marshal arguments (device, dtype, contiguity, shapes)
and pass raw device pointers plus torch's current HIP stream; every step of
the computation runs in the library's kernels.  There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "SwaError", "library_path", "load_library", "swa_attn_prefill",
    "swa_attn_verify_workspace_bytes", "swa_attn_verify", "swa_attn_verify_noalloc", "kv_ring_append",
    "swa_mtp_accept_workspace_bytes", "swa_mtp_greedy_accept", "swa_cache_advance",
    "swa_rope_apply", "rope_dims", "swa_attn_prefill_rope", "swa_attn_prefill_lse",
    "swa_attn_backward_workspace_bytes", "swa_attn_backward", "EXPORTED_SYMBOLS",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libswa_attn.so"
_lib = None

SWA_F32, SWA_BF16 = 0, 1
EXPORTED_SYMBOLS = ("swa_status_string", "swa_attn_prefill", "swa_attn_verify_workspace_bytes",
                    "swa_attn_verify", "kv_ring_append", "swa_mtp_accept_workspace_bytes",
                    "swa_mtp_greedy_accept", "swa_cache_advance", "swa_rope_apply",
                    "swa_attn_prefill_rope", "swa_attn_prefill_lse", "swa_attn_backward_workspace_bytes",
                    "swa_attn_backward", "swa_attn_verify_noalloc")


class SwaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, _LIB_NAME)


def load_library():
    """Load libswa_attn.so from the package directory (raises if absent)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m hybrid_sliding_window_swa_amd.build`")
    lib = ctypes.CDLL(path)
    i, p, f, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.swa_status_string.argtypes = [i]
    lib.swa_status_string.restype = ctypes.c_char_p
    lib.swa_attn_prefill.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p]
    lib.swa_attn_prefill.restype = i
    lib.swa_attn_verify_workspace_bytes.argtypes = [i, i, i, i, i, i, i, i, i]
    lib.swa_attn_verify_workspace_bytes.restype = sz
    lib.swa_attn_verify.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p, sz, p]
    lib.swa_attn_verify.restype = i
    lib.swa_attn_verify_noalloc.argtypes = [p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p]
    lib.swa_attn_verify_noalloc.restype = i
    lib.kv_ring_append.argtypes = [p, p, p, p, p, p, i, i, i, i, i, i, i, p]
    lib.kv_ring_append.restype = i
    i64 = ctypes.c_int64
    lib.swa_mtp_accept_workspace_bytes.argtypes = [i, i, i64]
    lib.swa_mtp_accept_workspace_bytes.restype = sz
    lib.swa_mtp_greedy_accept.argtypes = [p, p, p, p, i, i, i64, i, p, sz, p]
    lib.swa_mtp_greedy_accept.restype = i
    lib.swa_cache_advance.argtypes = [p, p, i, p]
    lib.swa_cache_advance.restype = i
    lib.swa_rope_apply.argtypes = [p, p, i, i, i, i, i, i, f, i, p]
    lib.swa_rope_apply.restype = i
    lib.swa_attn_prefill_rope.argtypes = [p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, f, i, p]
    lib.swa_attn_prefill_rope.restype = i
    lib.swa_attn_prefill_lse.argtypes = [p, p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p]
    lib.swa_attn_prefill_lse.restype = i
    lib.swa_attn_backward_workspace_bytes.argtypes = [i, i, i]
    lib.swa_attn_backward_workspace_bytes.restype = sz
    lib.swa_attn_backward.argtypes = [p, p, p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, i, i, f, i, p, sz, p]
    lib.swa_attn_backward.restype = i
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load_library().swa_status_string(status).decode()
        raise SwaError(status, f"{what}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, ndim=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    return t


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def swa_attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     sinks: Optional[torch.Tensor], window: int, q_offset: int = 0,
                     sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """Causal prefill: q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] (bf16 or fp32), sinks [Hq]
    fp32 or None; window <= 0 means global.  Returns o [B,Sq,Hq,D]."""
    lib = load_library()
    _dev(q, "q", ndim=4)
    _dev(k, "k", q.dtype, 4)
    _dev(v, "v", q.dtype, 4)
    _dev(sinks, "sinks", torch.float32, 1)
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("k/v shape mismatch")
    if sinks is not None and sinks.shape[0] != Hq:
        raise ValueError("sinks must have Hq entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", q.dtype, 4)
        if out.shape != q.shape:
            raise ValueError("out shape mismatch")
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    st = lib.swa_attn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out),
                              B, Sq, Sk, Hq, Hkv, D, int(window), int(q_offset), float(sm_scale),
                              _dtype_code(q), _stream(stream))
    _check(st, "swa_attn_prefill")
    return out


def swa_attn_prefill_rope(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          sinks: Optional[torch.Tensor], window: int, rot_dim: int, rope_base: float,
                          q_offset: int = 0, sm_scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Prefill with the queries rotated on load (q is only read; k must be
    rotated already).  Raises SwaError (unsupported) outside the
    sliding-window strip configurations."""
    lib = load_library()
    _dev(q, "q", ndim=4)
    _dev(k, "k", q.dtype, 4)
    _dev(v, "v", q.dtype, 4)
    _dev(sinks, "sinks", torch.float32, 1)
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("k/v shape mismatch")
    if sinks is not None and sinks.shape[0] != Hq:
        raise ValueError("sinks must have Hq entries")
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", q.dtype, 4)
        if out.shape != q.shape:
            raise ValueError("out shape mismatch")
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    st = lib.swa_attn_prefill_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(out), B, Sq, Sk, Hq, Hkv, D,
                                   int(window), int(q_offset), float(sm_scale), int(rot_dim),
                                   float(rope_base), _dtype_code(q), _stream(stream))
    _check(st, "swa_attn_prefill_rope")
    return out


def swa_attn_verify_workspace_bytes(B: int, q_len: int, Hq: int, Hkv: int, D: int,
                                    cache_slots: int, ring: bool, window: int,
                                    dtype: torch.dtype = torch.bfloat16) -> int:
    code = SWA_BF16 if dtype == torch.bfloat16 else SWA_F32
    return int(load_library().swa_attn_verify_workspace_bytes(B, q_len, Hq, Hkv, D, cache_slots,
                                                              int(bool(ring)), int(window), code))


def swa_attn_verify(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                    k_cache: torch.Tensor, v_cache: torch.Tensor, cache_len: torch.Tensor,
                    sinks: Optional[torch.Tensor], window: int, ring: bool,
                    sm_scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Verify q [B,T,Hq,D] (tokens at positions cache_len[b] + t) against the
    cache [B,slots,Hkv,D] (ring or linear) and the new rows k_new/v_new
    [B,T,Hkv,D].  cache_len: int32 [B] on the GPU.  Returns o [B,T,Hq,D]."""
    lib = load_library()
    _dev(q, "q", ndim=4)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, q.dtype, 4)
    _dev(cache_len, "cache_len", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    B, T, Hq, D = q.shape
    _, slots, Hkv, _ = k_cache.shape
    if k_new.shape != (B, T, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, q_len, Hkv, D]")
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    if cache_len.shape[0] != B:
        raise ValueError("cache_len must have B entries")
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    need = swa_attn_verify_workspace_bytes(B, T, Hq, Hkv, D, slots, ring, window, q.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", q.dtype, 4)
    st = lib.swa_attn_verify(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                             _ptr(cache_len), _ptr(sinks), _ptr(out), B, T, Hq, Hkv, D, slots,
                             int(bool(ring)), int(window), float(sm_scale), _dtype_code(q),
                             _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "swa_attn_verify")
    return out


def swa_attn_verify_noalloc(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                            k_cache: torch.Tensor, v_cache: torch.Tensor, cache_len: torch.Tensor,
                            sinks: Optional[torch.Tensor], window: int, ring: bool,
                            sm_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """swa_attn_verify with the split partials in the library's fixed
    per-GPU scratch (no workspace; calls on one GPU must not overlap).  With
    ``out`` given, the call allocates nothing."""
    lib = load_library()
    _dev(q, "q", ndim=4)
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, name, q.dtype, 4)
    _dev(cache_len, "cache_len", torch.int32, 1)
    _dev(sinks, "sinks", torch.float32, 1)
    B, T, Hq, D = q.shape
    _, slots, Hkv, _ = k_cache.shape
    if k_new.shape != (B, T, Hkv, D) or v_new.shape != k_new.shape:
        raise ValueError("k_new/v_new must be [B, q_len, Hkv, D]")
    if v_cache.shape != k_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shape mismatch")
    if cache_len.shape[0] != B:
        raise ValueError("cache_len must have B entries")
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    if out is None:
        out = torch.empty_like(q)
    else:
        _dev(out, "out", q.dtype, 4)
        if out.shape != q.shape:
            raise ValueError("out shape mismatch")
    st = lib.swa_attn_verify_noalloc(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(cache_len), _ptr(sinks), _ptr(out), B, T, Hq, Hkv, D, slots,
                                     int(bool(ring)), int(window), float(sm_scale), _dtype_code(q),
                                     _stream(stream))
    _check(st, "swa_attn_verify_noalloc")
    return out


def kv_ring_append(k_cache: torch.Tensor, v_cache: torch.Tensor, k_new: torch.Tensor,
                   v_new: torch.Tensor, cache_len: torch.Tensor, n_append: torch.Tensor,
                   ring: bool, stream=None) -> None:
    """Copy rows t < n_append[b] of k_new/v_new into the cache slots of
    positions cache_len[b] + t (ring: modulo the slot count).  In place."""
    lib = load_library()
    _dev(k_cache, "k_cache", ndim=4)
    _dev(v_cache, "v_cache", k_cache.dtype, 4)
    _dev(k_new, "k_new", k_cache.dtype, 4)
    _dev(v_new, "v_new", k_cache.dtype, 4)
    _dev(cache_len, "cache_len", torch.int32, 1)
    _dev(n_append, "n_append", torch.int32, 1)
    B, slots, Hkv, D = k_cache.shape
    T = k_new.shape[1]
    if k_new.shape != (B, T, Hkv, D) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    st = lib.kv_ring_append(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                            _ptr(cache_len), _ptr(n_append), B, T, Hkv, D, slots,
                            int(bool(ring)), _dtype_code(k_cache), _stream(stream))
    _check(st, "kv_ring_append")


def swa_mtp_accept_workspace_bytes(B: int, q_len: int, vocab: int) -> int:
    return int(load_library().swa_mtp_accept_workspace_bytes(B, q_len, vocab))


def swa_mtp_greedy_accept(logits: torch.Tensor, draft: Optional[torch.Tensor],
                          workspace: Optional[torch.Tensor] = None,
                          target: Optional[torch.Tensor] = None,
                          n_append: Optional[torch.Tensor] = None, stream=None):
    """Greedy draft acceptance: logits [B,q_len,vocab] (bf16 or fp32), draft
    [B,q_len-1] int32 (None when q_len == 1).  Returns (target [B,q_len]
    int32: per-row argmax, lowest index on ties; n_append [B] int32:
    1 + accepted leading drafts)."""
    lib = load_library()
    _dev(logits, "logits", ndim=3)
    B, T, V = logits.shape
    if draft is not None:
        _dev(draft, "draft", torch.int32, 2)
        if draft.shape != (B, T - 1):
            raise ValueError("draft must be [B, q_len - 1]")
    elif T > 1:
        raise ValueError("draft is required when q_len > 1")
    if target is None:
        target = torch.empty((B, T), dtype=torch.int32, device=logits.device)
    else:
        _dev(target, "target", torch.int32, 2)
        if target.shape != (B, T):
            raise ValueError("target must be [B, q_len]")
    if n_append is None:
        n_append = torch.empty((B,), dtype=torch.int32, device=logits.device)
    else:
        _dev(n_append, "n_append", torch.int32, 1)
        if n_append.shape[0] != B:
            raise ValueError("n_append must have B entries")
    need = swa_mtp_accept_workspace_bytes(B, T, V)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=logits.device)
    if workspace is not None:
        _dev(workspace, "workspace")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.swa_mtp_greedy_accept(_ptr(logits), _ptr(draft), _ptr(target), _ptr(n_append), B, T, V,
                                   _dtype_code(logits), _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "swa_mtp_greedy_accept")
    return target, n_append


def swa_cache_advance(cache_len: torch.Tensor, n_append: torch.Tensor, stream=None) -> None:
    """cache_len[b] += n_append[b] on the GPU (both int32 [B]).  In place."""
    lib = load_library()
    _dev(cache_len, "cache_len", torch.int32, 1)
    _dev(n_append, "n_append", torch.int32, 1)
    if n_append.shape != cache_len.shape:
        raise ValueError("cache_len and n_append must have the same length")
    st = lib.swa_cache_advance(_ptr(cache_len), _ptr(n_append), cache_len.shape[0], _stream(stream))
    _check(st, "swa_cache_advance")


def rope_dims(D: int, factor: float = 0.334) -> int:
    """Rotated dimensions per head for a partial-rotary factor: the largest
    even number <= factor * D (42 for D = 128 at the model's 0.334)."""
    return 2 * int(factor * D / 2)


def swa_rope_apply(x: torch.Tensor, rot_dim: int, base: float, pos0: Optional[torch.Tensor] = None,
                   pos_offset: int = 0, stream=None) -> torch.Tensor:
    """Rotate the first rot_dim dims of every head of x [B,S,H,D] in place;
    row s of request b is at position pos0[b] + pos_offset + s (pos0: int32
    [B] on the GPU, or None for 0).  Returns x."""
    lib = load_library()
    _dev(x, "x", ndim=4)
    _dev(pos0, "pos0", torch.int32, 1)
    B, S, H, D = x.shape
    if pos0 is not None and pos0.shape[0] != B:
        raise ValueError("pos0 must have B entries")
    st = lib.swa_rope_apply(_ptr(x), _ptr(pos0), int(pos_offset), B, S, H, D, int(rot_dim), float(base),
                            _dtype_code(x), _stream(stream))
    _check(st, "swa_rope_apply")
    return x


def swa_attn_prefill_lse(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: Optional[torch.Tensor],
                         window: int, q_offset: int = 0, sm_scale: Optional[float] = None, stream=None):
    """Training forward (bf16): returns (o [B,Sq,Hq,D], lse [B,Sq,Hq] fp32)."""
    lib = load_library()
    _dev(q, "q", torch.bfloat16, 4)
    _dev(k, "k", torch.bfloat16, 4)
    _dev(v, "v", torch.bfloat16, 4)
    _dev(sinks, "sinks", torch.float32, 1)
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D:
        raise ValueError("k/v shape mismatch")
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    o = torch.empty_like(q)
    lse = torch.empty((B, Sq, Hq), dtype=torch.float32, device=q.device)
    st = lib.swa_attn_prefill_lse(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o), _ptr(lse), B, Sq, Sk, Hq, Hkv,
                                  D, int(window), int(q_offset), float(sm_scale), SWA_BF16, _stream(stream))
    _check(st, "swa_attn_prefill_lse")
    return o, lse


def swa_attn_backward_workspace_bytes(B: int, Sq: int, Hq: int) -> int:
    return int(load_library().swa_attn_backward_workspace_bytes(B, Sq, Hq))


def swa_attn_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks: Optional[torch.Tensor],
                      o: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, window: int,
                      q_offset: int = 0, sm_scale: Optional[float] = None,
                      workspace: Optional[torch.Tensor] = None, stream=None):
    """Gradients of sum(dout * O) (bf16): returns (dq, dk, dv, dsink or None)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _dev(t, name, torch.bfloat16, 4)
    _dev(sinks, "sinks", torch.float32, 1)
    _dev(lse, "lse", torch.float32, 3)
    B, Sq, Hq, D = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    if v.shape != k.shape or Bk != B or Dk != D or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch")
    if lse.shape != (B, Sq, Hq):
        raise ValueError("lse must be [B, Sq, Hq]")
    if sm_scale is None:
        sm_scale = 1.0 / (D ** 0.5)
    need = int(lib.swa_attn_backward_workspace_bytes(B, Sq, Hq))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    dsink = None if sinks is None else torch.empty_like(sinks)
    st = lib.swa_attn_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(sinks), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq),
                               _ptr(dk), _ptr(dv), _ptr(dsink), B, Sq, Sk, Hq, Hkv, D, int(window), int(q_offset),
                               float(sm_scale), SWA_BF16, _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "swa_attn_backward")
    return dq, dk, dv, dsink
