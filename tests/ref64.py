"""Plain float64 definitions used to pin the oracle (not the oracle itself).

softmax with an optional sink term in the denominator (TransformerEngine PR
#678: a per-head learnable logit adds one exp term to the denominator), the
softmax vector-Jacobian product (RL-Kernel PR #453, "Fixed-order backward"),
and small numeric helpers (bf16 <-> fp32 bit views, ulps).
"""
import numpy as np

U = 2.0 ** -24          # unit roundoff of binary32
BF16_HALF_ULP_REL = 2.0 ** -8  # half an ulp, relative to a value at the bottom of its binade


def bf16_bits_to_f32(a):
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_torch(x):
    """Round binary32 -> bf16 (RNE) with torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return a.astype(np.float64)


def softmax64(x, sigma=None):
    """Row softmax of float64 ``x`` [rows, N]; ``sigma`` [rows] adds exp(sigma)
    to each row's denominator.  Returns (P, p_sink or None).  A row whose keys
    and sink are all -inf has no defined softmax; it returns P = 0 (and
    p_sink = 0), the convention the pages give for fully masked rows."""
    x = np.asarray(x, np.float64)
    rows, N = x.shape
    M = x.max(axis=1)
    if sigma is not None:
        sigma = np.asarray(sigma, np.float64)
        M = np.maximum(M, sigma)
    P = np.zeros_like(x)
    ps = np.zeros(rows) if sigma is not None else None
    ok = np.isfinite(M)
    with np.errstate(invalid="ignore", over="ignore"):
        ex = np.exp(x[ok] - M[ok, None])
        den = ex.sum(axis=1)
        if sigma is not None:
            es = np.exp(sigma[ok] - M[ok])
            den = den + es
            ps[ok] = es / den
        P[ok] = ex / den[:, None]
    return P, ps


def vjp64(P, g, p_sink=None):
    """float64 softmax VJP on given P, dP: delta = sum(P*dP), dS = P*(dP -
    delta); with a sink, d_sink share = -p_sink*delta."""
    P = np.asarray(P, np.float64)
    g = np.asarray(g, np.float64)
    delta = (P * g).sum(axis=1)
    dS = P * (g - delta[:, None])
    v = None if p_sink is None else -np.asarray(p_sink, np.float64) * delta
    return dS, delta, v


def bf16_ordered(bits):
    """Map bf16 bit patterns to integers ordered like the values, with +0 and
    -0 both mapped to 0."""
    b = np.asarray(bits, np.uint16).astype(np.int32)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def bf16_ulp_distance(a_bits, b_bits):
    return np.abs(bf16_ordered(a_bits) - bf16_ordered(b_bits))


def f32_ordered(x):
    b = np.asarray(x, np.float32).view(np.int32).astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b < 0, -mag, mag)
