"""Python binding of libjas.so: fixed-order, batch-invariant row softmax on
MI355X (gfx950).

The C ABI (include/jas.h) is the product; this module only marshals
arguments.  ``jas_fwd`` / ``jas_bwd`` / ``jas_fwd_ex`` / ``jas_bwd_ex`` /
``jas_bwd_workspace_bytes`` / ``jas_launch_plan`` / ``jas_status_str`` /
``jas_contract`` call the C functions of the same names with raw pointers.
``fwd`` and ``bwd`` take torch tensors: torch provides device memory and the current stream, every step of
the computation runs in the library's HIP kernels.  There is no fallback: if
``libjas.so`` is missing the first call raises.
"""
import ctypes
import os

__all__ = [
    "JAS_DTYPE_F32", "JAS_DTYPE_BF16", "JAS_DTYPE_F16", "JAS_FLAG_MASK", "JAS_FLAG_SINK",
    "JAS_FLAG_CAUSAL", "JAS_FLAG_KEY_LEN", "JAS_FLAG_LSE", "JAS_FLAG_PROBS", "JAS_FLAG_SCORES",
    "JAS_MAX_KEYS", "JAS_ATTN_MAX_KEYS",
    "STATUS", "JasError", "jas_desc_t", "jas_launch_t", "jas_attn_desc_t", "lib", "jas_fwd",
    "jas_fwd_ex", "jas_bwd", "jas_bwd_ex", "jas_bwd_noalloc", "jas_bwd_workspace_bytes",
    "jas_attn_fwd", "jas_attn_fwd_ex", "JAS_NOALLOC_MAX_ROWS",
    "jas_launch_plan", "jas_status_str", "jas_contract", "make_desc",
    "make_attn_desc", "fwd", "bwd", "fwd_prepared", "bwd_prepared", "attn_fwd",
    "attn_fwd_prepared", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjas.so")

JAS_DTYPE_F32, JAS_DTYPE_BF16, JAS_DTYPE_F16 = 0, 1, 2
JAS_FLAG_MASK, JAS_FLAG_SINK, JAS_FLAG_CAUSAL, JAS_FLAG_KEY_LEN, JAS_FLAG_LSE = 1, 2, 4, 8, 16
JAS_FLAG_PROBS, JAS_FLAG_SCORES = 32, 64
JAS_ATTN_MAX_KEYS = 16384
JAS_MAX_KEYS = 262144
JAS_NOALLOC_MAX_ROWS = 1048576
STATUS = {
    0: "JAS_OK", 1: "JAS_ERR_NULL_POINTER", 2: "JAS_ERR_BAD_SHAPE", 3: "JAS_ERR_BAD_DTYPE",
    4: "JAS_ERR_BAD_FLAGS", 5: "JAS_ERR_ALIASING", 6: "JAS_ERR_WORKSPACE",
    7: "JAS_ERR_UNSUPPORTED", 8: "JAS_ERR_HIP", 9: "JAS_ERR_ALIGNMENT", 10: "JAS_ERR_SCRATCH",
}


class jas_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("q_rows", ctypes.c_int64),
        ("keys", ctypes.c_int64), ("ld", ctypes.c_int64), ("dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32), ("mask_stride_b", ctypes.c_int64),
        ("mask_stride_h", ctypes.c_int64), ("mask_stride_q", ctypes.c_int64),
    ]


class jas_attn_desc_t(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("kv_heads", ctypes.c_int64),
        ("q_len", ctypes.c_int64), ("kv_len", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32), ("scale", ctypes.c_float),
        ("mask_stride_b", ctypes.c_int64), ("mask_stride_h", ctypes.c_int64),
        ("mask_stride_q", ctypes.c_int64),
    ]


class jas_launch_t(ctypes.Structure):
    _fields_ = [
        ("waves_per_row", ctypes.c_int32), ("chunks_per_lane", ctypes.c_int32),
        ("rows_per_block", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
        ("streaming", ctypes.c_int32), ("mask_in_registers", ctypes.c_int32),
    ]


class JasError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({jas_status_str(status)})")


_lib = None
_VP = ctypes.c_void_p
_DP = ctypes.POINTER(jas_desc_t)
_LP = ctypes.POINTER(jas_launch_t)


def lib():
    """Load libjas.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.jas_fwd.restype = ctypes.c_int
        L.jas_fwd.argtypes = [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.jas_fwd_ex.restype = ctypes.c_int
        L.jas_fwd_ex.argtypes = [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _LP, _VP]
        L.jas_bwd.restype = ctypes.c_int
        L.jas_bwd.argtypes = [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP]
        L.jas_bwd_ex.restype = ctypes.c_int
        L.jas_bwd_ex.argtypes = [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _LP,
                                 _VP]
        L.jas_bwd_noalloc.restype = ctypes.c_int
        L.jas_bwd_noalloc.argtypes = [_DP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.jas_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.jas_bwd_workspace_bytes.argtypes = [_DP]
        L.jas_launch_plan.restype = ctypes.c_int
        L.jas_launch_plan.argtypes = [_DP, ctypes.c_int, _LP, _LP]
        L.jas_status_str.restype = ctypes.c_char_p
        L.jas_status_str.argtypes = [ctypes.c_int]
        L.jas_contract.restype = ctypes.c_char_p
        L.jas_contract.argtypes = []
        _AP = ctypes.POINTER(jas_attn_desc_t)
        L.jas_attn_fwd.restype = ctypes.c_int
        L.jas_attn_fwd.argtypes = [_AP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]
        L.jas_attn_fwd_ex.restype = ctypes.c_int
        L.jas_attn_fwd_ex.argtypes = [_AP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                      ctypes.c_int, _VP]
        _lib = L
    return _lib


# ---- the C entry points, one to one -------------------------------------

def jas_fwd(desc, scores, mask, key_len, sink, probs, p_sink, lse, stream):
    return lib().jas_fwd(ctypes.byref(desc), scores, mask, key_len, sink, probs, p_sink, lse,
                         stream)


def jas_fwd_ex(desc, scores, mask, key_len, sink, probs, p_sink, lse, launch, stream):
    lp = ctypes.byref(launch) if launch is not None else None
    return lib().jas_fwd_ex(ctypes.byref(desc), scores, mask, key_len, sink, probs, p_sink, lse,
                            lp, stream)


def jas_bwd(desc, probs, dprobs, key_len, p_sink, dscores, d_sink, workspace, workspace_bytes,
            stream):
    return lib().jas_bwd(ctypes.byref(desc), probs, dprobs, key_len, p_sink, dscores, d_sink,
                         workspace, workspace_bytes, stream)


def jas_bwd_ex(desc, probs, dprobs, key_len, p_sink, dscores, d_sink, workspace, workspace_bytes,
               launch, stream):
    lp = ctypes.byref(launch) if launch is not None else None
    return lib().jas_bwd_ex(ctypes.byref(desc), probs, dprobs, key_len, p_sink, dscores, d_sink,
                            workspace, workspace_bytes, lp, stream)


def jas_bwd_noalloc(desc, probs, dprobs, key_len, p_sink, dscores, d_sink, stream):
    return lib().jas_bwd_noalloc(ctypes.byref(desc), probs, dprobs, key_len, p_sink, dscores,
                                 d_sink, stream)


def jas_bwd_workspace_bytes(desc):
    return int(lib().jas_bwd_workspace_bytes(ctypes.byref(desc)))


def jas_launch_plan(desc, backward, launch=None):
    """(status, jas_launch_t) of the geometry jas_fwd_ex / jas_bwd_ex would
    launch; host only."""
    plan = jas_launch_t()
    lp = ctypes.byref(launch) if launch is not None else None
    st = lib().jas_launch_plan(ctypes.byref(desc), int(backward), lp, ctypes.byref(plan))
    return st, plan


def jas_status_str(status):
    return lib().jas_status_str(int(status)).decode()


def jas_contract():
    return lib().jas_contract().decode()


# ---- torch-tensor marshalling -------------------------------------------

def _ptr(t):
    return None if t is None else t.data_ptr()


def _on_device(t, fn, *args):
    """Call a library entry point with ``t``'s device current and that
    device's current stream as the last argument, so that the launch goes
    to the device holding the tensors whatever device is current."""
    import torch
    with torch.cuda.device(t.device):
        return fn(*args, torch.cuda.current_stream(t.device).cuda_stream)


def make_desc(shape, dtype_code, flags=0, ld=None, mask_strides=(0, 0, 0)):
    B, H, S, N = (int(v) for v in shape)
    d = jas_desc_t()
    d.batch, d.heads, d.q_rows, d.keys = B, H, S, N
    d.ld = N if ld is None else int(ld)
    d.dtype = dtype_code
    d.flags = flags
    d.mask_stride_b, d.mask_stride_h, d.mask_stride_q = (int(v) for v in mask_strides)
    return d


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return JAS_DTYPE_BF16
    if t.dtype == torch.float32:
        return JAS_DTYPE_F32
    if t.dtype == torch.float16:
        return JAS_DTYPE_F16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _launch(launch):
    if launch is None:
        return None
    if isinstance(launch, jas_launch_t):
        return launch
    L = jas_launch_t()
    (L.waves_per_row, L.chunks_per_lane, L.rows_per_block, L.max_blocks, L.streaming,
     L.mask_in_registers) = (int(v) for v in (tuple(launch) + (0,) * 6)[:6])
    return L


def _shape4(t):
    if t.device.type != "cuda":
        raise ValueError(f"tensors must be in device memory, not on {t.device}")
    if t.dim() != 4:
        raise ValueError("tensors are [batch, heads, q_rows, keys]")
    B, H, S, N = t.shape
    bad = ValueError("rows must be contiguous with one row stride (ld)")
    if N > 1 and t.stride(3) != 1:
        raise bad
    # row r = (b*H + h)*S + q starts at element r*ld: each row dimension of
    # size above 1 must step by ld times the rows inside it (the stride of a
    # dimension of size 1 never addresses anything, and torch leaves it free)
    ld, inner = None, 1
    for dim in (2, 1, 0):
        if t.shape[dim] > 1:
            if ld is None:
                if t.stride(dim) % inner:
                    raise bad
                ld = t.stride(dim) // inner
            elif t.stride(dim) != inner * ld:
                raise bad
        inner *= t.shape[dim]
    ld = N if ld is None else ld
    if ld < N:
        raise bad
    return t.shape, ld


def _empty_rows_like(t, ld):
    """A tensor shaped like ``t`` whose rows have the same stride ``ld``."""
    import torch
    B, H, S, N = t.shape
    if ld == N:
        return torch.empty((B, H, S, N), dtype=t.dtype, device=t.device)
    flat = torch.empty(max(0, B * H * S * ld), dtype=t.dtype, device=t.device)
    return flat.view(B, H, S, ld)[..., :N]


def _check_out(out, like):
    if out.device != like.device:
        raise ValueError("every tensor must be on the scores' device")
    if out.shape != like.shape or out.dtype != like.dtype or \
            out.device.type != "cuda" or _shape4(out)[1] != _shape4(like)[1]:
        raise ValueError("the output must have the input's shape, dtype and row stride")


def _check_vec(t, like, dtype, count, name):
    """A side tensor (mask, sink, key lengths, per-row or per-head values,
    workspace): on ``like``'s device, of ``dtype``, contiguous, with at least
    ``count`` elements.  The library reads these through raw device
    pointers, so a host tensor or a short one must never reach it."""
    if t is None:
        return None
    if t.device != like.device:
        raise ValueError(f"{name} must be on the scores' device ({like.device}), not {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < count:
        raise ValueError(f"{name} needs at least {count} elements, has {t.numel()}")
    return t


def _fwd_args(scores, mask, mask_strides, sink, out, p_sink, launch, causal, key_len, lse,
              want_lse):
    """Validate a forward and allocate its missing outputs: (arguments of
    jas_fwd_ex without the stream, result tuple)."""
    import torch
    shape, ld = _shape4(scores)
    B, H, S, N = shape
    rows = B * H * S
    key_len = _check_vec(key_len, scores, torch.int32, B, "key_len")
    flags = (JAS_FLAG_CAUSAL if causal else 0) | (JAS_FLAG_KEY_LEN if key_len is not None else 0)
    if mask is not None:
        flags |= JAS_FLAG_MASK
        if mask_strides is None:
            m4 = mask.expand(B, H, S, N)
            if m4.stride(3) != 1:
                raise ValueError("mask keys must be contiguous")
            mask_strides = (m4.stride(0), m4.stride(1), m4.stride(2))
        if any(int(st) < 0 for st in mask_strides):
            raise ValueError("mask strides must be non-negative")
        mask_elems = 0 if rows == 0 else \
            sum((n - 1) * int(st) for n, st in zip(shape[:3], mask_strides)) + N
        _check_vec(mask, scores, torch.float32, mask_elems, "mask")
    if sink is not None:
        flags |= JAS_FLAG_SINK
        _check_vec(sink, scores, torch.float32, H, "sink")
    d = make_desc(shape, _dtype_code(scores), flags, ld, mask_strides or (0, 0, 0))
    if out is None:
        out = _empty_rows_like(scores, ld)
    _check_out(out, scores)
    if sink is not None and p_sink is None:
        p_sink = torch.empty(rows, dtype=torch.float32, device=scores.device)
    if sink is not None:
        _check_vec(p_sink, scores, torch.float32, rows, "p_sink")
    want_lse = want_lse or lse is not None
    if want_lse:
        d.flags |= JAS_FLAG_LSE
        if lse is None:
            lse = torch.empty(rows, dtype=torch.float32, device=scores.device)
        _check_vec(lse, scores, torch.float32, rows, "lse")
    args = (d, _ptr(scores), _ptr(mask), _ptr(key_len), _ptr(sink), _ptr(out),
            _ptr(p_sink) if sink is not None else None, _ptr(lse) if want_lse else None,
            _launch(launch))
    ps = p_sink if sink is not None else None
    return args, ((out, ps, lse) if want_lse else (out, ps))


def fwd(scores, mask=None, mask_strides=None, sink=None, out=None, p_sink=None, launch=None,
        causal=False, key_len=None, lse=None, want_lse=False):
    """Forward on device tensors.  ``scores`` [B,H,Sq,N] bf16/fp16/fp32 (rows
    may have a stride ld >= N); ``mask`` fp32 addressed with ``mask_strides``
    (b, h, q) in elements (default: a contiguous [B,H,Sq,N] tensor broadcast
    by its own zero strides); ``sink`` fp32 [H]; ``causal`` excludes keys past
    the causal condition; ``key_len`` int32 [B] excludes keys past each batch
    entry's length.  Returns (probs, p_sink), or (probs, p_sink, lse) when
    ``want_lse`` is set or an ``lse`` output (fp32 [B*H*Sq]) is given."""
    args, res = _fwd_args(scores, mask, mask_strides, sink, out, p_sink, launch, causal, key_len,
                          lse, want_lse)
    st = _on_device(scores, jas_fwd_ex, *args)
    if st != 0:
        raise JasError(st, "jas_fwd")
    return res


def fwd_prepared(scores, mask=None, mask_strides=None, sink=None, out=None, p_sink=None,
                 launch=None, causal=False, key_len=None, lse=None, want_lse=False):
    """:func:`fwd`'s checks and allocations done once: returns (run, result),
    where ``run()`` enqueues the same forward again on the same tensors with
    one call of jas_fwd_ex, on the stream current when this was called, and
    raises on an error status.  For loops that time the library, or that
    must not allocate; call ``run`` with the tensors' device current and
    keep the tensors alive while it is used."""
    import torch
    args, res = _fwd_args(scores, mask, mask_strides, sink, out, p_sink, launch, causal, key_len,
                          lse, want_lse)
    with torch.cuda.device(scores.device):
        stream = torch.cuda.current_stream(scores.device).cuda_stream
    return _prepared(lib().jas_fwd_ex, args, stream, "jas_fwd"), res


def _prepared(fn, args, stream, name):
    d, rest, launch = args[0], args[1:-1], args[-1]
    dp = ctypes.byref(d)
    lp = ctypes.byref(launch) if launch is not None else None
    keep = (d, launch)  # the structures the pointers above refer to

    def run():
        st = fn(dp, *rest, lp, stream)
        if st != 0:
            raise JasError(st, name)
    run.keep = keep
    return run


def _bwd_args(probs, dprobs, p_sink, out, d_sink, workspace, launch, causal, key_len):
    """Validate a backward and allocate its missing outputs: (arguments of
    jas_bwd_ex without the stream, result tuple)."""
    import torch
    shape, ld = _shape4(probs)
    B, H, S, N = shape
    key_len = _check_vec(key_len, probs, torch.int32, B, "key_len")
    flags = (JAS_FLAG_SINK if p_sink is not None else 0) | (JAS_FLAG_CAUSAL if causal else 0) | \
        (JAS_FLAG_KEY_LEN if key_len is not None else 0)
    d = make_desc(shape, _dtype_code(probs), flags, ld)
    _check_out(dprobs, probs)
    if out is None:
        out = _empty_rows_like(probs, ld)
    _check_out(out, probs)
    ws_bytes = jas_bwd_workspace_bytes(d)
    if p_sink is not None:
        _check_vec(p_sink, probs, torch.float32, B * H * S, "p_sink")
        if d_sink is None:
            d_sink = torch.empty(H, dtype=torch.float32, device=probs.device)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device=probs.device)
        _check_vec(d_sink, probs, torch.float32, H, "d_sink")
        _check_vec(workspace, probs, torch.uint8, ws_bytes, "workspace")
    args = (d, _ptr(probs), _ptr(dprobs), _ptr(key_len), _ptr(p_sink), _ptr(out),
            _ptr(d_sink) if p_sink is not None else None,
            _ptr(workspace) if p_sink is not None else None,
            workspace.numel() if workspace is not None else 0, _launch(launch))
    return args, (out, (d_sink if p_sink is not None else None))


def bwd(probs, dprobs, p_sink=None, out=None, d_sink=None, workspace=None, launch=None,
        causal=False, key_len=None):
    """Backward on device tensors (``causal`` / ``key_len`` as for the
    forward: P is taken as +0 on excluded keys).  Returns (dscores, d_sink or
    None)."""
    args, res = _bwd_args(probs, dprobs, p_sink, out, d_sink, workspace, launch, causal, key_len)
    st = _on_device(probs, jas_bwd_ex, *args)
    if st != 0:
        raise JasError(st, "jas_bwd")
    return res


def bwd_prepared(probs, dprobs, p_sink=None, out=None, d_sink=None, workspace=None, launch=None,
                 causal=False, key_len=None):
    """:func:`bwd` prepared once, as :func:`fwd_prepared`: returns (run,
    result)."""
    import torch
    args, res = _bwd_args(probs, dprobs, p_sink, out, d_sink, workspace, launch, causal, key_len)
    with torch.cuda.device(probs.device):
        stream = torch.cuda.current_stream(probs.device).cuda_stream
    return _prepared(lib().jas_bwd_ex, args, stream, "jas_bwd"), res


# ---- fused attention ----------------------------------------------------------

def make_attn_desc(B, H, Hkv, Sq, N, D, dtype_code, flags=0, scale=1.0, mask_strides=(0, 0, 0)):
    d = jas_attn_desc_t()
    d.batch, d.heads, d.kv_heads, d.q_len, d.kv_len, d.head_dim = (
        int(v) for v in (B, H, Hkv, Sq, N, D))
    d.dtype = dtype_code
    d.flags = flags
    d.scale = float(scale)
    d.mask_stride_b, d.mask_stride_h, d.mask_stride_q = (int(v) for v in mask_strides)
    return d


def jas_attn_fwd(desc, q, k, v, mask, key_len, sink, out, lse, p_sink, probs, scores, stream):
    return lib().jas_attn_fwd(ctypes.byref(desc), q, k, v, mask, key_len, sink, out, lse, p_sink,
                              probs, scores, stream)


def jas_attn_fwd_ex(desc, q, k, v, mask, key_len, sink, out, lse, p_sink, probs, scores,
                    query_blocks, stream):
    return lib().jas_attn_fwd_ex(ctypes.byref(desc), q, k, v, mask, key_len, sink, out, lse,
                                 p_sink, probs, scores, query_blocks, stream)


def _attn_tensor(t, name, like=None):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory, not on {t.device}")
    if t.dim() != 4 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [batch, heads, len, head_dim] tensor")
    if like is not None and (t.device != like.device or t.dtype != like.dtype):
        raise ValueError(f"{name} must match q's device and dtype")
    return t


def _attn_args(q, k, v, scale, mask, mask_strides, sink, causal, key_len, want_lse, want_probs,
               want_scores, out, query_blocks):
    """Validate a fused attention call and allocate its outputs: (arguments
    of jas_attn_fwd_ex without the stream, result dict)."""
    import math
    import torch
    _attn_tensor(q, "q")
    _attn_tensor(k, "k", q)
    _attn_tensor(v, "v", q)
    B, H, Sq, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    if tuple(v.shape) != tuple(k.shape) or Bk != B or Dk != D:
        raise ValueError("k and v must be [batch, kv_heads, kv_len, head_dim] like q")
    if q.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("attention takes bf16 or fp16")
    rows = B * H * Sq
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    key_len = _check_vec(key_len, q, torch.int32, B, "key_len")
    flags = (JAS_FLAG_CAUSAL if causal else 0) | (JAS_FLAG_KEY_LEN if key_len is not None else 0)
    if mask is not None:
        flags |= JAS_FLAG_MASK
        if mask_strides is None:
            m4 = mask.expand(B, H, Sq, N)
            if m4.stride(3) != 1:
                raise ValueError("mask keys must be contiguous")
            mask_strides = (m4.stride(0), m4.stride(1), m4.stride(2))
        if any(int(st) < 0 for st in mask_strides):
            raise ValueError("mask strides must be non-negative")
        mask_elems = 0 if rows == 0 else \
            sum((n - 1) * int(st) for n, st in zip((B, H, Sq), mask_strides)) + N
        _check_vec(mask, q, torch.float32, mask_elems, "mask")
    if sink is not None:
        flags |= JAS_FLAG_SINK
        _check_vec(sink, q, torch.float32, H, "sink")
    res = {"out": None, "lse": None, "p_sink": None, "probs": None, "scores": None}
    dev = q.device
    if want_lse:
        flags |= JAS_FLAG_LSE
        res["lse"] = torch.empty(rows, dtype=torch.float32, device=dev)
    if sink is not None:
        res["p_sink"] = torch.empty(rows, dtype=torch.float32, device=dev)
    if want_probs:
        flags |= JAS_FLAG_PROBS
        res["probs"] = torch.empty((B, H, Sq, N), dtype=q.dtype, device=dev)
    if want_scores:
        flags |= JAS_FLAG_SCORES
        res["scores"] = torch.empty((B, H, Sq, N), dtype=torch.float32, device=dev)
    d = make_attn_desc(B, H, Hkv, Sq, N, D, _dtype_code(q), flags, scale, mask_strides or (0, 0, 0))
    if out is None:
        out = torch.empty_like(q)
    _attn_tensor(out, "out", q)
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    res["out"] = out
    args = (d, _ptr(q), _ptr(k), _ptr(v), _ptr(mask), _ptr(key_len), _ptr(sink), _ptr(out),
            _ptr(res["lse"]), _ptr(res["p_sink"]), _ptr(res["probs"]), _ptr(res["scores"]),
            int(query_blocks))
    return args, res


def attn_fwd(q, k, v, scale=None, mask=None, mask_strides=None, sink=None, causal=False,
             key_len=None, want_lse=False, want_probs=False, want_scores=False, out=None,
             query_blocks=0):
    """Fused attention forward on device tensors: q [B, H, Sq, D], k and v
    [B, Hkv, N, D] (bf16 or fp16, contiguous), ``scale`` (default
    1/sqrt(D)).  Mask, sink, causal and key lengths as for :func:`fwd`.
    Returns a dict with ``out`` and, when asked (or a sink is given),
    ``lse``, ``p_sink``, ``probs``, ``scores``.  ``query_blocks`` (0, 1 or 2)
    is the launch's 16-query blocks per wavefront, 0 = the library's choice;
    it never changes the results."""
    args, res = _attn_args(q, k, v, scale, mask, mask_strides, sink, causal, key_len, want_lse,
                           want_probs, want_scores, out, query_blocks)
    st = _on_device(q, jas_attn_fwd_ex, *args)
    if st != 0:
        raise JasError(st, "jas_attn_fwd")
    return res


def attn_fwd_prepared(q, k, v, scale=None, mask=None, mask_strides=None, sink=None, causal=False,
                      key_len=None, want_lse=False, want_probs=False, want_scores=False, out=None,
                      query_blocks=0):
    """:func:`attn_fwd` prepared once, as :func:`fwd_prepared`: returns (run,
    result dict); ``run()`` is one call of jas_attn_fwd_ex on the same
    tensors."""
    import torch
    args, res = _attn_args(q, k, v, scale, mask, mask_strides, sink, causal, key_len, want_lse,
                           want_probs, want_scores, out, query_blocks)
    with torch.cuda.device(q.device):
        stream = torch.cuda.current_stream(q.device).cuda_stream
    L = lib()
    d, rest = args[0], args[1:]
    dp = ctypes.byref(d)

    def run():
        st = L.jas_attn_fwd_ex(dp, *rest, stream)
        if st != 0:
            raise JasError(st, "jas_attn_fwd")
    run.keep = d
    return run, res
