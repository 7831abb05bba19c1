"""Helpers for the GPU parity tests: comparisons at the stated tolerance and
row sampling.  Tolerances (the acceptance bar for this softmax): bf16 and
fp16 results within 1 ulp of their type of the oracle (+0 and -0 equal),
fp32 results within 4e-6 relative (absolute floor 1e-38 for subnormal
results); the row log-sum-exp within 4e-6 * max(1, |lse|); stage-isolated
backward results bit-exact."""
import numpy as np
import torch

import oracle
import synth
from tests.ref64 import bf16_ulp_distance

F32_RTOL = 4e-6
F32_ATOL = 1e-38


def dev():
    return torch.device("cuda:0")


def log(msg):
    print(msg, flush=True)


def assert_close(got, want, what=""):
    """got/want: numpy bit views (uint16 bf16, float16 or float32)."""
    assert got.shape == want.shape and got.dtype == want.dtype, what
    if got.dtype == np.float16:  # sign-magnitude 16 bits: the bf16 ordering applies
        got, want = got.view(np.uint16), want.view(np.uint16)
    if got.dtype == np.uint16:
        d = bf16_ulp_distance(got, want)
        bad = np.count_nonzero(d > 1)
        assert bad == 0, f"{what}: {bad} values differ by more than 1 bf16 ulp (max {int(d.max())})"
        return int(d.max()) if d.size else 0
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    lim = F32_RTOL * np.abs(want.astype(np.float64)) + F32_ATOL
    bad = np.count_nonzero(~(err <= lim))
    assert bad == 0, f"{what}: {bad} fp32 values outside 4e-6 relative (worst {np.max(err / lim):.3g}x)"
    return float(np.max(err / lim)) if err.size else 0.0


def assert_bitexact(got, want, what=""):
    assert got.shape == want.shape, what
    g = got.view(np.uint16 if got.itemsize == 2 else np.uint32)
    w = want.view(np.uint16 if want.itemsize == 2 else np.uint32)
    bad = np.count_nonzero(g != w)
    assert bad == 0, f"{what}: {bad} values not bit-identical"


LSE_TOL = 4e-6


def assert_lse_close(got, want, what="lse"):
    """Row log-sum-exp: -inf exactly where the oracle has -inf, elsewhere
    within 4e-6 * max(1, |lse|) (the hardware logarithm and the GPU's
    exponentials inside L against the oracle's)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, what
    ninf = np.isneginf(want)
    assert np.array_equal(np.isneginf(got), ninf), f"{what}: -inf rows differ"
    g, w = got[~ninf].astype(np.float64), want[~ninf].astype(np.float64)
    err = np.abs(g - w)
    lim = LSE_TOL * np.maximum(1.0, np.abs(w))
    bad = np.count_nonzero(~(err <= lim))
    assert bad == 0, f"{what}: {bad} values outside tolerance (worst {np.max(err / lim):.3g}x)"
    return float(np.max(err / lim)) if err.size else 0.0


def sample_rows(rows, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.unique(np.concatenate([[0, rows - 1], rng.choice(rows, size=min(k, rows), replace=False)]))
    return idx.astype(np.int64)


def gather_rows(t4, idx):
    """Host numpy bits of rows `idx` of a [B,H,S,N] device tensor."""
    N = t4.shape[-1]
    flat = t4.reshape(-1, N)
    sel = flat.index_select(0, torch.as_tensor(idx, device=t4.device))
    return synth.to_numpy_bits(sel)


def oracle_rows_fwd(s_rows, N, mask_rows=None, sigma_rows=None):
    """Oracle forward on k independent rows (as k heads of one query)."""
    k = s_rows.shape[0]
    P, ps = oracle.fwd(s_rows.reshape(1, k, 1, N), 1, k, 1, N, mask=mask_rows,
                       mask_strides=(0, N, 0), sink=sigma_rows)
    return P.reshape(k, N), ps


def oracle_rows_bwd(P_rows, g_rows, N, ps_rows=None):
    k = P_rows.shape[0]
    dS, v = oracle.bwd(P_rows.reshape(1, k, 1, N), g_rows.reshape(1, k, 1, N), 1, k, 1, N,
                       p_sink=ps_rows)
    return dS.reshape(k, N), v
