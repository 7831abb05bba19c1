"""Pins for the oracle's forward pass.

Against the float64 definition of softmax (with the sink's exp term in the
denominator, TransformerEngine PR #678) under an error bound derived from the
binary32 roundings the fixed-order method takes (RL-Kernel PR #453,
Fixed-order online softmax), plus special cases whose binary32 result is
exact, and the indexing rules: mask by broadcast strides, sink by head only.
"""
import math

import numpy as np
import pytest

import oracle as O
from tests.ref64 import U, bf16_bits_to_f32, softmax64, f32_to_bf16_bits_torch

E0 = abs(float(O.log2e()) * math.log(2.0) - 1.0)
TILE = 256


def eta(z):
    """Relative error of exp_(fl(z)) against exp(z): the difference, the
    product with log2e, the error of log2e itself, the final rounding."""
    return np.abs(z) * (2 * U + E0) + U


def fwd_rel_bound(x, sigma=None):
    """Per-element relative error bound of the fixed-order forward pass
    against float64 softmax, for binary32 inputs x [N] (already masked)."""
    x = np.asarray(x, np.float64)
    N = x.size
    T = (N + TILE - 1) // TILE
    xp = np.full(T * TILE, -np.inf)
    xp[:N] = x
    xt = xp.reshape(T, TILE)
    m = xt.max(axis=1)
    with np.errstate(invalid="ignore"):
        ej = np.where(np.isfinite(xt), eta(xt - m[:, None]), 0.0)
    eta_l = np.where(np.isfinite(m), ej.max(axis=1), 0.0) + 8 * U
    M = -np.inf
    eps = 0.0
    for t in range(T):
        Mn = max(M, m[t])
        if Mn == -np.inf:
            continue
        ea = eta(M - Mn) if M != -np.inf else 0.0
        eb = eta(m[t] - Mn) if m[t] != -np.inf else 0.0
        eps = max(eps + ea + U, eta_l[t] + eb + U) + U
        M = Mn
    if sigma is not None and sigma != -np.inf:
        Mn = max(M, sigma)
        ea = eta(M - Mn) if M != -np.inf else 0.0
        eps = max(eps + ea + U, eta(sigma - Mn) + U) + U
        M = Mn
    eps_inv = eps + U
    with np.errstate(invalid="ignore"):
        ec = np.where(np.isfinite(m), eta(m - M), 0.0)
    per = (ej + ec[:, None] + eps_inv + 2 * U).reshape(-1)[:N] * 1.01
    ps = None if sigma is None or sigma == -np.inf else (eta(sigma - M) + eps_inv + U) * 1.01
    return per, ps


def masked_x(scores_f32, mask):
    x = scores_f32.astype(np.float32)
    if mask is not None:
        x = (x + mask.astype(np.float32)).astype(np.float32)
    return x


def check_rows_against_float64(Pout, ps_out, x, sigma, bf16_out):
    rows, N = x.shape
    Pref, psref = softmax64(x.astype(np.float64), None if sigma is None else sigma.astype(np.float64))
    Pgot = bf16_bits_to_f32(Pout).astype(np.float64) if bf16_out else Pout.astype(np.float64)
    for r in range(rows):
        rel, rel_ps = fwd_rel_bound(x[r], None if sigma is None else float(sigma[r]))
        bound = rel * Pref[r] + 2.0 ** -126
        if bf16_out:
            bound = bound + 2.0 ** -8 * (Pref[r] + bound)  # half a bf16 ulp
        err = np.abs(Pgot[r] - Pref[r])
        assert np.all(err <= bound), (r, np.max(err / np.maximum(bound, 1e-300)))
        if sigma is not None:
            b = (rel_ps if rel_ps is not None else 0.0) * psref[r] + 2.0 ** -126
            assert abs(float(ps_out[r]) - psref[r]) <= b, (r, ps_out[r], psref[r])


def to_bf16(x):
    return f32_to_bf16_bits_torch(x)


@pytest.mark.parametrize("N", [1, 7, 255, 256, 257, 513, 1000, 4352])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_mask,with_sink", [(False, False), (True, False), (False, True), (True, True)])
def test_fwd_matches_float64_softmax(N, dtype, with_mask, with_sink):
    rng = np.random.default_rng(N * 7 + (dtype == "bf16") + 2 * with_mask + 4 * with_sink)
    rows = 6
    s32 = (rng.standard_normal((rows, N)) * 3).astype(np.float32)
    s32[0, rng.integers(0, N, max(1, N // 100))] *= 8  # a few outliers
    if dtype == "bf16":
        s = to_bf16(s32)
        sf = bf16_bits_to_f32(s)
    else:
        s = s32
        sf = s32
    mask = None
    if with_mask:
        mask = np.where(rng.random((rows, N)) < 0.2, -np.inf, rng.standard_normal((rows, N))).astype(np.float32)
        mask[1, :] = -np.inf                  # a fully masked row
        if N > 300:
            mask[2, 256:512] = -np.inf        # a fully masked tile
    sink = None
    sig_rows = None
    if with_sink:
        sink = (rng.standard_normal(rows) * 2).astype(np.float32)
        sig_rows = sink
    # rows as heads (B=1, H=rows, Sq=1): sink is per head, mask row stride N
    P, ps = O.fwd(s.reshape(1, rows, 1, N), 1, rows, 1, N, mask=mask,
                  mask_strides=(0, N, 0), sink=sink)
    x = masked_x(sf, mask)
    check_rows_against_float64(P.reshape(rows, N), ps, x, sig_rows, dtype == "bf16")
    # rows sum to 1 - p_sink (or 0 for a fully masked row without sink)
    Pf = bf16_bits_to_f32(P) if dtype == "bf16" else P
    sums = Pf.reshape(rows, N).astype(np.float64).sum(axis=1)
    target = np.ones(rows) - (ps.astype(np.float64) if ps is not None else 0)
    if not with_sink:
        target[np.all(np.isneginf(x), axis=1)] = 0.0   # fully masked rows
    tol = (2.0 ** -8 if dtype == "bf16" else 1e-5)
    assert np.all(np.abs(sums - target) <= tol), (sums, target)


@pytest.mark.parametrize("N", [1, 2, 255, 256, 257, 4352, 8449])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_uniform_row_is_exact(N, dtype):
    # every e is 1, every tile sum and the merged sum are exact integers, so
    # P = fl(1/N); with a sink equal to the row value, P = p_sink = fl(1/(N+1))
    val = np.float32(0.375)
    s = np.full((1, 1, 1, N), val, np.float32)
    if dtype == "bf16":
        s = to_bf16(s)
    P, _ = O.fwd(s, 1, 1, 1, N)
    want = np.float32(1.0) / np.float32(N)
    Pf = bf16_bits_to_f32(P) if dtype == "bf16" else P
    if dtype == "bf16":
        assert np.all(P == to_bf16(np.array([want], np.float32))[0])
    else:
        assert np.all(Pf == want)
    P2, ps = O.fwd(s, 1, 1, 1, N, sink=np.array([val], np.float32))
    want2 = np.float32(1.0) / np.float32(N + 1)
    assert ps[0] == want2
    if dtype == "f32":
        assert np.all(P2 == want2)


def test_single_key_one_hot_and_masked_rows():
    P, _ = O.fwd(np.array([[[[3.5]]]], np.float32), 1, 1, 1, 1)
    assert P.reshape(-1)[0] == 1.0
    x = np.full(600, -np.inf, np.float32)
    x[437] = -12.25
    P, _ = O.fwd(x.reshape(1, 1, 1, -1), 1, 1, 1, 600)
    P = P.reshape(-1)
    assert P[437] == 1.0 and np.count_nonzero(P) == 1
    # fully masked row: P = 0, and with a sink p_sink = 1
    s = np.random.default_rng(0).standard_normal(600).astype(np.float32).reshape(1, 1, 1, -1)
    mask = np.full(600, -np.inf, np.float32)
    P, _ = O.fwd(s, 1, 1, 1, 600, mask=mask)
    assert np.all(P == 0) and not np.any(np.signbit(P))
    P, ps = O.fwd(s, 1, 1, 1, 600, mask=mask, sink=np.array([0.7], np.float32))
    assert np.all(P == 0) and ps[0] == 1.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_minus_inf_sink_equals_no_sink_and_inf_key_equals_masked_key(dtype):
    rng = np.random.default_rng(9)
    N = 777
    s32 = (rng.standard_normal(N) * 2).astype(np.float32)
    s32[[5, 300, 700]] = -np.inf
    s = to_bf16(s32) if dtype == "bf16" else s32
    s = s.reshape(1, 1, 1, N)
    P0, _ = O.fwd(s, 1, 1, 1, N)
    P1, ps = O.fwd(s, 1, 1, 1, N, sink=np.array([-np.inf], np.float32))
    assert P0.tobytes() == P1.tobytes() and ps[0] == 0.0
    # the same -inf keys expressed as a mask on finite scores
    s2 = s32.copy()
    s2[[5, 300, 700]] = 1.5
    mask = np.zeros(N, np.float32)
    mask[[5, 300, 700]] = -np.inf
    s2 = to_bf16(s2) if dtype == "bf16" else s2
    P2, _ = O.fwd(s2.reshape(1, 1, 1, N), 1, 1, 1, N, mask=mask)
    assert P0.tobytes() == P2.tobytes()


def test_exact_shift_invariance():
    # scores on a grid of multiples of 2^-8 in [-16, 16]: every difference is
    # exact, so adding 16 to the whole row (and to the sink) changes no bit
    rng = np.random.default_rng(4)
    N = 1100
    s = (rng.integers(-4096, 4097, N) / 256.0).astype(np.float32)
    P0, ps0 = O.fwd(s.reshape(1, 1, 1, N), 1, 1, 1, N, sink=np.array([0.5], np.float32))
    P1, ps1 = O.fwd((s + np.float32(16)).reshape(1, 1, 1, N), 1, 1, 1, N,
                    sink=np.array([16.5], np.float32))
    assert P0.tobytes() == P1.tobytes() and ps0.tobytes() == ps1.tobytes()


def test_indexing_mask_strides_and_sink_per_head():
    # sink indexed by head only (one value per head, shape [H]); the mask is
    # addressed b*msb + h*msh + q*msq + k.  Reference rows are assembled here
    # by explicit loops.
    rng = np.random.default_rng(21)
    B, H, Sq, N = 2, 3, 4, 300
    s = (rng.standard_normal((B, H, Sq, N)) * 2).astype(np.float32)
    sink = np.array([-1.0, 0.5, 2.0], np.float32)
    for layout in ["full", "batch_key", "head_key", "query_key"]:
        if layout == "full":
            mask = np.where(rng.random((B, H, Sq, N)) < 0.3, -np.inf, 0.25).astype(np.float32)
            strides = (H * Sq * N, Sq * N, N)
            get = lambda b, h, q: mask[b, h, q]
        elif layout == "batch_key":
            mask = np.where(rng.random((B, N)) < 0.3, -np.inf, -0.5).astype(np.float32)
            strides = (N, 0, 0)
            get = lambda b, h, q: mask[b]
        elif layout == "head_key":
            mask = np.where(rng.random((H, N)) < 0.3, -np.inf, 1.0).astype(np.float32)
            strides = (0, N, 0)
            get = lambda b, h, q: mask[h]
        else:
            mask = np.where(rng.random((Sq, N)) < 0.3, -np.inf, 0.0).astype(np.float32)
            strides = (0, 0, N)
            get = lambda b, h, q: mask[q]
        P, ps = O.fwd(s, B, H, Sq, N, mask=mask, mask_strides=strides, sink=sink)
        P = P.reshape(B, H, Sq, N)
        ps = ps.reshape(B, H, Sq)
        for b in range(B):
            for h in range(H):
                for q in range(Sq):
                    x = (s[b, h, q] + get(b, h, q)).astype(np.float32)
                    Pref, psref = softmax64(x[None].astype(np.float64), np.array([float(sink[h])]))
                    assert np.allclose(P[b, h, q], Pref[0], rtol=5e-6, atol=1e-30), (layout, b, h, q)
                    assert abs(ps[b, h, q] - psref[0]) <= 5e-6 * psref[0] + 1e-30


def test_row_stride_ld_reads_and_writes_only_the_row():
    rng = np.random.default_rng(8)
    rows, N, ld = 5, 300, 320
    s = np.full((rows, ld), np.nan, np.float32)     # padding must never be read
    s[:, :N] = rng.standard_normal((rows, N)).astype(np.float32)
    P, _ = O.fwd(s, 1, 1, rows, N, ld=ld)
    assert not np.any(np.isnan(P[:, :N]))
    assert np.all(P[:, N:] == 0)                    # never written
    P2, _ = O.fwd(np.ascontiguousarray(s[:, :N]), 1, 1, rows, N)
    assert P[:, :N].tobytes() == P2.tobytes()


def test_thread_count_does_not_change_bytes():
    rng = np.random.default_rng(12)
    s = (rng.standard_normal((2, 3, 7, 531)) * 3).astype(np.float32)
    sink = rng.standard_normal(3).astype(np.float32)
    a, pa = O.fwd(s, 2, 3, 7, 531, sink=sink, threads=1)
    b, pb = O.fwd(s, 2, 3, 7, 531, sink=sink, threads=5)
    assert a.tobytes() == b.tobytes() and pa.tobytes() == pb.tobytes()
