"""CPU oracle for sliding-window / global attention with per-head sinks.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg import this package; the GPU library and its
Python binding never do.  It shares no code with the GPU path.

The arithmetic lives in ``oracle.c`` (plain C, fp64, two-pass softmax with
the sink in the denominator); this module builds it with gcc if needed and
marshals numpy / torch arrays into it.  Every output is float64.

Parity pins (checked by the CPU tests against things other than the oracle
itself): torch's scaled-dot-product attention in fp64 with a sink column and
with band / causal masks, closed forms for W=1 and for Q=0 with one-hot
values, the sigmoid(LSE - sink) identity, weights + sink mass = 1, GQA vs
repeated KV heads, verify vs successive single-token decodes and vs prefill
rows, chunked vs unchunked prefill, and hand-derived golden values.  The
greedy draft acceptance is pinned by hand-built cases (the release blog's
accept, accept, reject, discard example among them), tie breaking and
numpy's argmax.  The partial rotary embedding is pinned by closed forms
(one-hot inputs at known angles), position 0 as the identity, composition of
rotations, preserved pair norms and the relative-position property of the
rotated dot product.  The backward is pinned by central finite differences
of the forward oracle, by torch fp64 autograd through scaled-dot-product
attention with the sink column, and by the sink-gradient identity
dsink_h = -sum_i p_sink,i <dO_i, O_i>.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORC_OK, ORC_BAD_ARGS, ORC_HISTORY_SHORT, ORC_NO_MEMORY = 0, 1, 2, 3


def build(src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _bind(lib):
    c_f = ctypes.POINTER(ctypes.c_float)
    c_d = ctypes.POINTER(ctypes.c_double)
    c_i64 = ctypes.POINTER(ctypes.c_int64)
    c_u8 = ctypes.POINTER(ctypes.c_uint8)
    i, l, d = ctypes.c_int, ctypes.c_long, ctypes.c_double
    lib.oracle_prefill.argtypes = [c_f, c_f, c_f, c_d, c_d, c_d, c_d, c_d,
                                   i, i, i, i, i, i, i, i, d]
    lib.oracle_prefill.restype = i
    lib.oracle_prefill_rows.argtypes = [c_f, c_i64, l, c_f, c_f, l, l, c_d, c_d,
                                        i, i, i, i, l, d]
    lib.oracle_prefill_rows.restype = i
    lib.oracle_verify.argtypes = [c_f, c_f, c_f, c_f, c_f, c_i64, c_i64, c_d, c_d,
                                  i, i, i, i, i, l, i, d]
    lib.oracle_verify.restype = i
    lib.oracle_ring_append.argtypes = [c_u8, c_u8, c_u8, c_u8, c_i64, c_i64,
                                       i, i, i, i, l, i, i]
    lib.oracle_ring_append.restype = i
    lib.oracle_greedy_accept.argtypes = [c_f, ctypes.POINTER(ctypes.c_int32), i, i, l,
                                         ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
    lib.oracle_greedy_accept.restype = i
    lib.oracle_prefill_backward.argtypes = [c_f, c_f, c_f, c_d, c_f, c_d, c_d, c_d, c_d,
                                            i, i, i, i, i, i, i, i, d]
    lib.oracle_prefill_backward.restype = i
    lib.oracle_rope.argtypes = [c_d, c_d, c_i64, l, i, i, i, d]
    lib.oracle_rope.restype = i
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i
    return lib


def load(path: str = None):
    """Load (building first if absent) and return the ctypes library."""
    global _lib
    with _lock:
        if path is not None:
            return _bind(ctypes.CDLL(path))
        if _lib is None:
            if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
                build()
            _lib = _bind(ctypes.CDLL(_LIB_PATH))
        return _lib


def num_threads() -> int:
    return load().oracle_num_threads()


# ---------------------------------------------------------------- marshalling

def _f32(x) -> np.ndarray:
    """fp32 C-contiguous numpy copy of a torch tensor / array (exact for bf16)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float32).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _i64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _nullable_d(a):
    return None if a is None else _p(a, ctypes.c_double)


def _check(rc: int, what: str):
    if rc != ORC_OK:
        raise ValueError(f"oracle {what} failed with code {rc}")


# ---------------------------------------------------------------- entry points

def prefill(q, k, v, sinks=None, window: int = 0, q_offset: int = 0, scale: float = None,
            want_lse: bool = False, want_psink: bool = False, want_weights: bool = False):
    """Attention of q [B,Sq,Hq,D] over k/v [B,Sk,Hkv,D]; row r at position q_offset + r.

    Returns O [B,Sq,Hq,D] float64, or a dict with "o" plus the requested
    "lse" / "psink" [B,Sq,Hq] and "weights" [B,Sq,Hq,Sk]."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    assert k.shape == v.shape and k.shape[0] == B and k.shape[3] == D
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = None if sinks is None else _f64(sinks)
    o = np.empty((B, Sq, Hq, D), np.float64)
    lse = np.empty((B, Sq, Hq), np.float64) if want_lse else None
    ps = np.empty((B, Sq, Hq), np.float64) if want_psink else None
    w = np.empty((B, Sq, Hq, Sk), np.float64) if want_weights else None
    rc = load().oracle_prefill(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                               _nullable_d(s), _p(o, ctypes.c_double), _nullable_d(lse),
                               _nullable_d(ps), _nullable_d(w),
                               B, Sq, Sk, Hq, Hkv, D, int(window), int(q_offset), float(scale))
    _check(rc, "prefill")
    if not (want_lse or want_psink or want_weights):
        return o
    out = {"o": o}
    if want_lse:
        out["lse"] = lse
    if want_psink:
        out["psink"] = ps
    if want_weights:
        out["weights"] = w
    return out


def prefill_rows(q_rows, rows, k, v, sinks=None, window: int = 0, q_offset: int = 0,
                 scale: float = None, k_base: int = 0):
    """Selected rows of one request: q_rows [n,Hq,D] for query rows ``rows``;
    k/v [nk,Hkv,D] hold positions k_base.. .  Returns O [n,Hq,D] float64."""
    q_rows, k, v = _f32(q_rows), _f32(k), _f32(v)
    rows = _i64(rows)
    n, Hq, D = q_rows.shape
    nk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = None if sinks is None else _f64(sinks)
    o = np.empty((n, Hq, D), np.float64)
    rc = load().oracle_prefill_rows(_p(q_rows, ctypes.c_float), _p(rows, ctypes.c_int64), n,
                                    _p(k, ctypes.c_float), _p(v, ctypes.c_float), int(k_base), nk,
                                    _nullable_d(s), _p(o, ctypes.c_double),
                                    Hq, Hkv, D, int(window), int(q_offset), float(scale))
    _check(rc, "prefill_rows")
    return o


def verify(q, k_new, v_new, k_hist, v_hist, hist_base, cache_len, sinks=None,
           window: int = 0, scale: float = None):
    """q [B,T,Hq,D] at positions L_b..L_b+T-1 over the logical history
    k_hist/v_hist [B,Hlen,Hkv,D] (row r = position hist_base[b] + r) and the
    new rows k_new/v_new [B,T,Hkv,D].  Returns O [B,T,Hq,D] float64."""
    q, k_new, v_new = _f32(q), _f32(k_new), _f32(v_new)
    k_hist, v_hist = _f32(k_hist), _f32(v_hist)
    hist_base, cache_len = _i64(hist_base), _i64(cache_len)
    B, T, Hq, D = q.shape
    _, Hlen, Hkv, _ = k_hist.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = None if sinks is None else _f64(sinks)
    o = np.empty((B, T, Hq, D), np.float64)
    rc = load().oracle_verify(_p(q, ctypes.c_float), _p(k_new, ctypes.c_float), _p(v_new, ctypes.c_float),
                              _p(k_hist, ctypes.c_float), _p(v_hist, ctypes.c_float),
                              _p(hist_base, ctypes.c_int64), _p(cache_len, ctypes.c_int64),
                              _nullable_d(s), _p(o, ctypes.c_double),
                              B, T, Hq, Hkv, D, Hlen, int(window), float(scale))
    _check(rc, "verify")
    return o


def prefill_backward(q, k, v, dout, sinks=None, window: int = 0, q_offset: int = 0, scale: float = None):
    """Gradients of sum(dout * prefill(q, k, v, sinks)): returns (dq, dk, dv,
    dsink) as float64 (dsink [Hq], zeros when sinks is None)."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    assert dout.shape == q.shape and v.shape == k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    s = None if sinks is None else _f64(sinks)
    dq = np.empty(q.shape, np.float64)
    dk = np.empty(k.shape, np.float64)
    dv = np.empty(k.shape, np.float64)
    ds = np.zeros((Hq,), np.float64)
    rc = load().oracle_prefill_backward(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                                        _nullable_d(s), _p(dout, ctypes.c_float), _p(dq, ctypes.c_double),
                                        _p(dk, ctypes.c_double), _p(dv, ctypes.c_double), _p(ds, ctypes.c_double),
                                        B, Sq, Sk, Hq, Hkv, D, int(window), int(q_offset), float(scale))
    _check(rc, "prefill_backward")
    return dq, dk, dv, ds


def ring_append(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
                cache_len, n_append, ring: bool):
    """In-place commit of accepted rows into numpy caches [B,slots,Hkv,D]
    (any dtype; copied bytewise).  k_new/v_new [B,T,Hkv,D] of the same dtype."""
    for a in (k_cache, v_cache, k_new, v_new):
        assert isinstance(a, np.ndarray) and a.flags.c_contiguous
    assert k_cache.dtype == k_new.dtype == v_cache.dtype == v_new.dtype
    B, slots, Hkv, D = k_cache.shape
    T = k_new.shape[1]
    cl, na = _i64(cache_len), _i64(n_append)
    u8 = ctypes.c_uint8
    rc = load().oracle_ring_append(_p(k_cache.view(np.uint8), u8), _p(v_cache.view(np.uint8), u8),
                                   _p(k_new.view(np.uint8), u8), _p(v_new.view(np.uint8), u8),
                                   _p(cl, ctypes.c_int64), _p(na, ctypes.c_int64),
                                   B, T, Hkv, D, slots, int(bool(ring)), k_cache.dtype.itemsize)
    _check(rc, "ring_append")


def greedy_accept(logits, draft):
    """Greedy acceptance of drafts: logits [B,T,V] (any float dtype, upcast to
    fp32), draft [B,T-1] int.  Returns (target [B,T] int32: argmax with the
    lowest index among equal maxima, n_append [B] int32: 1 + accepted drafts)."""
    lg = _f32(logits)
    B, T, V = lg.shape
    dr = np.ascontiguousarray(np.asarray(draft.cpu() if hasattr(draft, "cpu") else draft), dtype=np.int32)
    assert dr.shape == (B, T - 1)
    target = np.empty((B, T), dtype=np.int32)
    n_append = np.empty((B,), dtype=np.int32)
    rc = load().oracle_greedy_accept(_p(lg, ctypes.c_float), _p(dr, ctypes.c_int32), B, T, V,
                                     _p(target, ctypes.c_int32), _p(n_append, ctypes.c_int32))
    _check(rc, "greedy_accept")
    return target, n_append


def rope_dims(D: int, factor: float = 0.334) -> int:
    """Rotated dimensions per head: the largest even number <= factor * D."""
    return 2 * int(factor * D / 2)


def rope(x, positions, rot: int, base: float):
    """Partial rotary embedding of x [..., H, D] (leading dims flattened to
    rows; positions broadcast to them).  Returns float64 of x's shape."""
    xd = _f64(x)
    shape = xd.shape
    H, D = shape[-2], shape[-1]
    rows = int(np.prod(shape[:-2])) if len(shape) > 2 else 1
    pos = np.ascontiguousarray(np.broadcast_to(_i64(positions), shape[:-2]).reshape(-1), dtype=np.int64)
    assert pos.shape[0] == rows
    xd = np.ascontiguousarray(xd.reshape(rows, H, D))
    out = np.empty_like(xd)
    rc = load().oracle_rope(_p(xd, ctypes.c_double), _p(out, ctypes.c_double), _p(pos, ctypes.c_int64),
                            rows, H, D, int(rot), float(base))
    _check(rc, "rope")
    return out.reshape(shape)
