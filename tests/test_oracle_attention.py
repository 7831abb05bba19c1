"""Pins for the oracle's fixed-order attention forward (QK, the row softmax,
PV).

RL-Kernel PR #240, Fixed Reduction Contract: each score accumulates the head
dimension in ascending order, each output element accumulates the keys in
ascending order; RL-Kernel PR #453, Summary: the softmax sits between the QK
GEMM and the AV GEMM and rounds P once to the tensor dtype.  Checked
against float64 attention under a bound derived from the roundings, against
the softmax oracle on its own scores (byte for byte), and on cases with a
closed form: one-hot attention returns a value row exactly, equal keys give
the mean of the values, grouped key/value heads equal repeated heads.
"""
import numpy as np
import pytest

import oracle as O
from tests.ref64 import f32_to_bf16_bits_torch, softmax64

U = 2.0 ** -24


def as_f64(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def cast(x32, dt):
    return f32_to_bf16_bits_torch(x32) if dt == "bf16" else x32.astype(np.float16)


def draw(seed, B, H, Hkv, Sq, N, D, dt, std=1.0):
    rng = np.random.default_rng(seed)
    q = cast((rng.standard_normal((B, H, Sq, D)) * std).astype(np.float32), dt)
    k = cast((rng.standard_normal((B, Hkv, N, D)) * std).astype(np.float32), dt)
    v = cast(rng.standard_normal((B, Hkv, N, D)).astype(np.float32), dt)
    return q, k, v


def ref64(q, k, v, scale, mask=None, sink=None, vis=None):
    """float64 attention: S = scale q k^T, P = softmax(S + mask) with the
    sink in the denominator and hidden keys removed, O = P V."""
    B, H, Sq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    g = H // Hkv
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    S = np.zeros((B, H, Sq, N))
    P = np.zeros((B, H, Sq, N))
    Oo = np.zeros((B, H, Sq, D))
    absS = np.zeros((B, H, Sq, N))
    for b in range(B):
        for h in range(H):
            kk, vv = kf[b, h // g], vf[b, h // g]
            S[b, h] = scale * (qf[b, h] @ kk.T)
            absS[b, h] = abs(scale) * (np.abs(qf[b, h]) @ np.abs(kk).T)
            x = S[b, h] + (0.0 if mask is None else mask[b])
            if vis is not None:
                x = np.where(vis[b], x, -np.inf)
            sig = None if sink is None else np.full(Sq, float(sink[h]))
            P[b, h], _ = softmax64(x, sig)
            Oo[b, h] = P[b, h] @ vv
    return S, absS, P, Oo


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("case", ["plain", "mask_sink", "causal_keylen", "gqa"])
def test_attention_against_float64(dt, case):
    B, H, Hkv, Sq, N, D = 2, 4, 4, 9, 600, 64
    if case == "gqa":
        Hkv = 2
    q, k, v = draw(11, B, H, Hkv, Sq, N, D, dt, std=0.8)
    scale = np.float32(1.0 / np.sqrt(D))
    mask = sink = kl = None
    causal = False
    vis = None
    if case == "mask_sink":
        mask = np.zeros((B, N), np.float32)
        mask[1, 500:] = -np.inf
        mask[0, :7] = -2.5
        sink = np.array([0.3, -1.0, 2.0, 0.0], np.float32)
    if case == "causal_keylen":
        causal = True
        kl = np.array([600, 350], np.int32)
        qq = np.arange(Sq)[:, None]
        kk = np.arange(N)[None, :]
        vis = [(kk <= (N - Sq) + qq) & (kk < kl[b]) for b in range(B)]
    r = O.attn_fwd(q, k, v, scale, mask=mask, mask_strides=(N, 0, 0), causal=causal,
                   key_len=kl, sink=sink, want_probs=True, want_scores=True)
    S64, absS, P64, O64 = ref64(q, k, v, float(scale), mask=mask, sink=sink, vis=vis)
    # scores: two fp32 roundings orders apart at most D*u*sum|q_d k_d| (plus the scale)
    assert np.all(np.abs(r["scores"] - S64) <= (D + 2) * U * absS + 1e-30)
    # output: P rounded to the dtype (relative 2^-8 for bf16, 2^-11 for fp16),
    # sums of exact products in fp32, one final rounding
    eps = 2.0 ** -8 if dt == "bf16" else 2.0 ** -11
    vabs = np.zeros_like(O64)
    g = H // Hkv
    for b in range(B):
        for h in range(H):
            vabs[b, h] = P64[b, h] @ np.abs(as_f64(v)[b, h // g])
    got = as_f64(r["out"])
    assert np.all(np.abs(got - O64) <= eps * (vabs + np.abs(O64)) + 1e-6 * vabs + 1e-30)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_probabilities_are_the_softmax_of_the_scores(dt):
    # P is the row softmax oracle applied to the binary32 scores, rounded once
    B, H, Sq, N, D = 1, 2, 7, 513, 128
    q, k, v = draw(12, B, H, H, Sq, N, D, dt)
    sink = np.array([0.5, -0.5], np.float32)
    r = O.attn_fwd(q, k, v, np.float32(0.088), sink=sink, causal=True, want_probs=True,
                   want_scores=True)
    P32, ps, lse = O.fwd(r["scores"], B, H, Sq, N, sink=sink, causal=True, want_lse=True)
    want = cast(P32, dt)
    assert r["probs"].view(np.uint16).tobytes() == want.view(np.uint16).tobytes()
    assert r["p_sink"].tobytes() == ps.tobytes() and r["lse"].tobytes() == lse.tobytes()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_one_hot_attention_returns_a_value_row_exactly(dt):
    # q = 16 e_0, key 5 = 8 e_0, other keys -8 e_0: scores 128 and -128, the
    # others' exponentials flush to +0, P is exactly one-hot, O = V[5]
    B, H, Sq, N, D = 1, 1, 3, 300, 64
    q = np.zeros((B, H, Sq, D), np.float32)
    q[..., 0] = 16.0
    k = np.zeros((B, H, N, D), np.float32)
    k[..., 0] = -8.0
    k[0, 0, 5, 0] = 8.0
    v = np.random.default_rng(13).standard_normal((B, H, N, D)).astype(np.float32)
    q, k, v = cast(q, dt), cast(k, dt), cast(v, dt)
    r = O.attn_fwd(q, k, v, np.float32(1.0), want_probs=True)
    P = as_f64(r["probs"])[0, 0]
    assert np.all(P[:, 5] == 1.0) and np.count_nonzero(P) == Sq
    for i in range(Sq):
        assert r["out"][0, 0, i].view(np.uint16).tobytes() == v[0, 0, 5].view(np.uint16).tobytes()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_equal_keys_give_the_mean_of_the_values(dt):
    B, H, Sq, N, D = 1, 1, 2, 256, 64
    q, _, v = draw(14, B, H, H, Sq, N, D, dt)
    k1 = cast(np.random.default_rng(15).standard_normal((1, 1, 1, D)).astype(np.float32), dt)
    k = np.ascontiguousarray(np.broadcast_to(k1, (B, H, N, D)))
    r = O.attn_fwd(q, k, v, np.float32(0.125), want_probs=True)
    P = as_f64(r["probs"])
    assert np.all(P == P[0, 0, 0, 0])                # uniform: one rounded value 1/256
    mean = (as_f64(v)[0, 0] * P[0, 0, 0, 0]).sum(axis=0)
    eps = 2.0 ** -8 if dt == "bf16" else 2.0 ** -11
    got = as_f64(r["out"])[0, 0]
    assert np.all(np.abs(got - mean) <= eps * np.abs(mean) + 1e-5)


def test_grouped_heads_equal_repeated_heads():
    B, H, Hkv, Sq, N, D = 2, 6, 2, 5, 300, 64
    q, k, v = draw(16, B, H, Hkv, Sq, N, D, "bf16")
    kr = np.ascontiguousarray(np.repeat(k, H // Hkv, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, H // Hkv, axis=1))
    a = O.attn_fwd(q, k, v, np.float32(0.1))
    b = O.attn_fwd(q, kr, vr, np.float32(0.1))
    assert a["out"].tobytes() == b["out"].tobytes() and a["lse"].tobytes() == b["lse"].tobytes()


def test_rows_are_independent():
    # a query computed alone gives the bytes it gets among others
    B, H, Sq, N, D = 1, 2, 6, 400, 64
    q, k, v = draw(17, B, H, H, Sq, N, D, "bf16")
    full = O.attn_fwd(q, k, v, np.float32(0.1), causal=False)
    part = O.attn_fwd(np.ascontiguousarray(q[:, :, 2:3]), k, v, np.float32(0.1))
    assert part["out"].tobytes() == np.ascontiguousarray(full["out"][:, :, 2:3]).tobytes()
