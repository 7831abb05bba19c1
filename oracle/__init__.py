"""CPU oracle for the fixed-order row softmax -- TEST INFRASTRUCTURE ONLY.

This package wraps ``libjas_oracle.so`` (built from ``jas_oracle.c`` by
``oracle/build.py``) with numpy arrays.  It is the reference the HIP library is
checked against.  Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import it; the HIP library and its Python
binding never do.

Arrays: bf16 tensors travel as ``numpy.uint16`` bit patterns, fp16 tensors as
``numpy.float16``, fp32 tensors as ``numpy.float32``.  All functions follow the pages cited in ``jas_oracle.c``:
RL-Kernel PR #453 (fixed-order online softmax, fixed-order backward), ROCm
TransformerEngine PR #678 (softmax sink), RL-Kernel PR #240 (fixed power-of-two
reduction tree, fully masked rows, the row log-sum-exp, FP16 beside BF16).
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libjas_oracle.so")
_lib = None

F32, BF16, F16 = 0, 1, 2
_I64 = ctypes.c_int64
_VP = ctypes.c_void_p


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.jas_oracle_fwd.restype = ctypes.c_int
        L.jas_oracle_fwd.argtypes = [ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _VP, _VP,
                                     _I64, _I64, _I64, ctypes.c_int, _VP, _VP, _VP, _VP, _VP,
                                     ctypes.c_int]
        L.jas_oracle_bwd.restype = ctypes.c_int
        L.jas_oracle_bwd.argtypes = [ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _VP, _VP,
                                     ctypes.c_int, _VP, _VP, _VP, _VP, ctypes.c_int]
        L.jas_oracle_attn_fwd.restype = ctypes.c_int
        L.jas_oracle_attn_fwd.argtypes = [ctypes.c_int, _I64, _I64, _I64, _I64, _I64, _I64, _VP,
                                          _VP, _VP, ctypes.c_float, _VP, _I64, _I64, _I64,
                                          ctypes.c_int, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          ctypes.c_int]
        L.jas_oracle_dsink.restype = ctypes.c_int
        L.jas_oracle_dsink.argtypes = [_I64, _I64, _I64, _VP, _VP]
        L.jas_oracle_exp.restype = ctypes.c_float
        L.jas_oracle_exp.argtypes = [ctypes.c_float]
        L.jas_oracle_log2e.restype = ctypes.c_float
        L.jas_oracle_log2e.argtypes = []
        L.jas_oracle_bf16.restype = ctypes.c_uint16
        L.jas_oracle_bf16.argtypes = [ctypes.c_float]
        L.jas_oracle_f16_array.restype = None
        L.jas_oracle_f16_array.argtypes = [_VP, _VP, _I64]
        L.jas_oracle_f16_decode_array.restype = None
        L.jas_oracle_f16_decode_array.argtypes = [_VP, _VP, _I64]
        L.jas_oracle_tree_sum256.restype = ctypes.c_float
        L.jas_oracle_tree_sum256.argtypes = [_VP]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"scores must be float32, float16 or uint16 (bf16 bits), got {a.dtype}")


def _key_len(key_len, B):
    if key_len is None:
        return None
    k = np.ascontiguousarray(key_len, dtype=np.int32)
    if k.size < B:
        raise ValueError("key_len needs one value per batch entry")
    return k


def fwd(scores, B, H, Sq, N, ld=None, mask=None, mask_strides=(0, 0, 0), sink=None,
        threads=None, causal=False, key_len=None, want_lse=False):
    """Forward pass.  ``scores`` is a C-contiguous array holding B*H*Sq rows of
    stride ``ld`` (default N).  ``causal`` excludes keys past the causal
    condition, ``key_len`` (int32 [B]) keys past each batch entry's length.
    Returns ``(P, p_sink)``, or ``(P, p_sink, lse)`` with ``want_lse``; ``P``
    has the layout and dtype of ``scores`` (row padding past N is left zero),
    ``p_sink`` is float32 [B*H*Sq] or None when no sink is given, ``lse`` the
    float32 [B*H*Sq] row log-sum-exp."""
    scores = np.ascontiguousarray(scores)
    ld = N if ld is None else ld
    rows = B * H * Sq
    if scores.size < (rows - 1) * ld + N if rows else 0:
        raise ValueError("scores too small for the shape")
    P = np.zeros_like(scores)
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.float32)
    if sink is not None:
        sink = np.ascontiguousarray(sink, dtype=np.float32)
        if sink.size < H:
            raise ValueError("sink needs one value per head")
    ps = np.zeros(rows, np.float32) if sink is not None else None
    lse = np.zeros(rows, np.float32) if want_lse else None
    msb, msh, msq = mask_strides
    kl = _key_len(key_len, B)
    rc = lib().jas_oracle_fwd(_dtype_code(scores), B, H, Sq, N, ld, _ptr(scores), _ptr(mask),
                              msb, msh, msq, int(bool(causal)), _ptr(kl), _ptr(sink), _ptr(P),
                              _ptr(ps), _ptr(lse), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"jas_oracle_fwd failed: {rc}")
    return (P, ps, lse) if want_lse else (P, ps)


def bwd(P, dP, B, H, Sq, N, ld=None, p_sink=None, threads=None, causal=False, key_len=None):
    """Backward pass on stored probabilities (P taken as +0 on keys the
    ``causal`` / ``key_len`` exclusion removes).  Returns ``(dS, v)`` where
    ``v`` is the float32 per-row d_sink share (None without ``p_sink``)."""
    P = np.ascontiguousarray(P)
    dP = np.ascontiguousarray(dP)
    if P.dtype != dP.dtype or P.shape != dP.shape:
        raise ValueError("P and dP must share dtype and shape")
    ld = N if ld is None else ld
    rows = B * H * Sq
    dS = np.zeros_like(P)
    v = None
    if p_sink is not None:
        p_sink = np.ascontiguousarray(p_sink, dtype=np.float32)
        v = np.zeros(rows, np.float32)
    kl = _key_len(key_len, B)
    rc = lib().jas_oracle_bwd(_dtype_code(P), B, H, Sq, N, ld, _ptr(P), _ptr(dP),
                              int(bool(causal)), _ptr(kl), _ptr(p_sink), _ptr(dS), _ptr(v),
                              threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"jas_oracle_bwd failed: {rc}")
    return dS, v


def attn_fwd(q, k, v, scale, mask=None, mask_strides=(0, 0, 0), causal=False, key_len=None,
             sink=None, want_probs=False, want_scores=False, threads=None):
    """Fixed-order attention forward.  q [B, H, Sq, D], k and v [B, Hkv, N, D]
    (uint16 bf16 bits or float16), ``scale`` the binary32 score scale.
    Returns a dict with ``out`` [B, H, Sq, D] (dtype of q), ``lse`` and
    ``p_sink`` (float32 [B*H*Sq], p_sink None without a sink) and, when asked,
    ``probs`` [B, H, Sq, N] (dtype of q) and ``scores`` (float32)."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if q.dtype != k.dtype or q.dtype != v.dtype or k.shape != v.shape:
        raise ValueError("q, k, v must share a dtype; k and v a shape")
    B, H, Sq, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    if Bk != B or Dk != D or H % Hkv:
        raise ValueError("shapes do not match")
    dt = _dtype_code(q)
    if dt == F32:
        raise TypeError("attention inputs are bf16 or fp16")
    rows = B * H * Sq
    out = np.zeros_like(q)
    lse = np.zeros(rows, np.float32)
    ps = np.zeros(rows, np.float32) if sink is not None else None
    probs = np.zeros((B, H, Sq, N), q.dtype) if want_probs else None
    scores = np.zeros((B, H, Sq, N), np.float32) if want_scores else None
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.float32)
    if sink is not None:
        sink = np.ascontiguousarray(sink, dtype=np.float32)
    kl = _key_len(key_len, B)
    msb, msh, msq = mask_strides
    rc = lib().jas_oracle_attn_fwd(dt, B, H, Hkv, Sq, N, D, _ptr(q), _ptr(k), _ptr(v),
                                   float(np.float32(scale)), _ptr(mask), msb, msh, msq,
                                   int(bool(causal)), _ptr(kl), _ptr(sink), _ptr(out), _ptr(lse),
                                   _ptr(ps), _ptr(probs), _ptr(scores), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"jas_oracle_attn_fwd failed: {rc}")
    return {"out": out, "lse": lse, "p_sink": ps, "probs": probs, "scores": scores}


def dsink(v, B, H, Sq):
    """Per-head d_sink from per-row shares ``v`` (float32 [B*H*Sq])."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.zeros(H, np.float32)
    rc = lib().jas_oracle_dsink(B, H, Sq, _ptr(v), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"jas_oracle_dsink failed: {rc}")
    return out


def exp_(y: float) -> np.float32:
    return np.float32(lib().jas_oracle_exp(float(np.float32(y))))


def log2e() -> np.float32:
    return np.float32(lib().jas_oracle_log2e())


def bf16_rne(x: float) -> int:
    return int(lib().jas_oracle_bf16(float(np.float32(x))))


def f16_rne(x):
    """binary32 array -> binary16 bit patterns (uint16), the oracle's rounding."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().jas_oracle_f16_array(_ptr(x), _ptr(out), x.size)
    return out


def f16_decode(h):
    """binary16 bit patterns (uint16) -> binary32, the oracle's widening."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().jas_oracle_f16_decode_array(_ptr(h), _ptr(out), h.size)
    return out


def tree_sum256(v) -> np.float32:
    v = np.ascontiguousarray(v, dtype=np.float32)
    if v.size != 256:
        raise ValueError("tree_sum256 takes exactly 256 values")
    return np.float32(lib().jas_oracle_tree_sum256(_ptr(v)))
