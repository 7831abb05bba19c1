"""Pins for causal and key-length exclusion in the oracle.

The causal condition is RL-Kernel PR #240's (Prefill / Decode: a key is
visible to a query when key_index <= Skv - Sq + query_index); key padding
with fully masked rows is the same page's Path Status.  An excluded key must
behave exactly like a key whose score is -inf: the forward with exclusion is
compared byte for byte with the forward on an explicit -inf mask built here
from the condition, and with float64 softmax over the visible keys.  The
backward takes P as +0 on excluded keys without reading it.
"""
import numpy as np
import pytest

import oracle as O
from tests.ref64 import f32_to_bf16_bits_torch, softmax64


def causal_mask(Sq, N):
    q = np.arange(Sq)[:, None]
    k = np.arange(N)[None, :]
    return np.where(k <= (N - Sq) + q, 0.0, -np.inf).astype(np.float32)


@pytest.mark.parametrize("Sq,N", [(300, 300), (64, 600), (40, 40), (9, 513), (600, 300)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causal_equals_explicit_minus_inf_mask(Sq, N, dtype):
    rng = np.random.default_rng(Sq * 3 + N)
    B, H = 2, 2
    s32 = (rng.standard_normal((B, H, Sq, N)) * 2).astype(np.float32)
    s = f32_to_bf16_bits_torch(s32) if dtype == "bf16" else s32
    sink = rng.standard_normal(H).astype(np.float32)
    P1, ps1 = O.fwd(s, B, H, Sq, N, causal=True, sink=sink)
    P2, ps2 = O.fwd(s, B, H, Sq, N, mask=causal_mask(Sq, N), mask_strides=(0, 0, N), sink=sink)
    assert P1.tobytes() == P2.tobytes() and ps1.tobytes() == ps2.tobytes()
    # float64: softmax over the visible keys of each query
    x = (s32 if dtype == "f32" else
         (s.astype(np.uint32) << 16).view(np.float32)).reshape(B * H, Sq, N).astype(np.float64)
    for r in range(B * H):
        xm = x[r] + causal_mask(Sq, N)
        Pref, psref = softmax64(xm, np.full(Sq, float(sink[r % H])))
        Pg = P1.reshape(B * H, Sq, N)[r]
        Pg = Pg if dtype == "f32" else (Pg.astype(np.uint32) << 16).view(np.float32)
        tol = 2.0 ** -8 if dtype == "bf16" else 2e-6
        assert np.allclose(Pg, Pref, rtol=tol, atol=1e-30)
    # a query with no visible key (Sq > N): P = 0, p_sink = 1
    if Sq > N:
        assert np.all(P1.reshape(B * H, Sq, N)[:, 0] == 0)
        assert np.all(ps1.reshape(B * H, Sq)[:, 0] == 1.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_key_len_equals_padding_mask(dtype):
    rng = np.random.default_rng(17)
    B, H, Sq, N = 4, 2, 7, 700
    kl = np.array([700, 513, 0, 1000], np.int32)  # full, partial tile, empty, clamped
    s32 = (rng.standard_normal((B, H, Sq, N)) * 2).astype(np.float32)
    s = f32_to_bf16_bits_torch(s32) if dtype == "bf16" else s32
    mask = np.zeros((B, N), np.float32)
    for b in range(B):
        mask[b, max(0, min(int(kl[b]), N)):] = -np.inf
    P1, _ = O.fwd(s, B, H, Sq, N, key_len=kl)
    P2, _ = O.fwd(s, B, H, Sq, N, mask=mask, mask_strides=(N, 0, 0))
    assert P1.tobytes() == P2.tobytes()
    assert np.all(P1.reshape(B, H, Sq, N)[2] == 0)
    # both exclusions together cut at the shorter prefix
    P3, _ = O.fwd(s, B, H, Sq, N, key_len=kl, causal=True)
    m2 = mask[:, None, None, :] + causal_mask(Sq, N)[None, None]
    P4, _ = O.fwd(s, B, H, Sq, N, mask=np.ascontiguousarray(np.broadcast_to(m2, (B, H, Sq, N))),
                  mask_strides=(H * Sq * N, Sq * N, N))
    assert P3.tobytes() == P4.tobytes()


def test_negative_key_len_is_an_empty_row():
    s = np.ones((1, 1, 3, 300), np.float32)
    P, ps = O.fwd(s, 1, 1, 3, 300, key_len=np.array([-5], np.int32), sink=np.zeros(1, np.float32))
    assert np.all(P == 0) and np.all(ps == 1.0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_takes_excluded_p_as_zero(dtype):
    # with exclusion, whatever P holds past the visible prefix is not read:
    # the result equals the backward on P with +0 written there
    rng = np.random.default_rng(5)
    B, H, Sq, N = 2, 3, 33, 600
    kl = np.array([600, 257], np.int32)
    P32 = (np.abs(rng.standard_normal((B, H, Sq, N))) / N).astype(np.float32)
    g32 = rng.standard_normal((B, H, Sq, N)).astype(np.float32)
    P, g = ((f32_to_bf16_bits_torch(P32), f32_to_bf16_bits_torch(g32)) if dtype == "bf16"
            else (P32, g32))
    ps = rng.random(B * H * Sq).astype(np.float32)
    dS1, v1 = O.bwd(P, g, B, H, Sq, N, p_sink=ps, causal=True, key_len=kl)
    Pz = P.copy().reshape(B, H, Sq, N)
    q = np.arange(Sq)[:, None]
    k = np.arange(N)[None, :]
    for b in range(B):
        vis = (k <= (N - Sq) + q) & (k < kl[b])
        Pz[b][:, ~vis] = 0
    dS2, v2 = O.bwd(Pz, g, B, H, Sq, N, p_sink=ps)
    assert dS1.tobytes() == dS2.tobytes() and v1.tobytes() == v2.tobytes()
    # and the signed zeros of the excluded region come from dP - delta
    d = dS1.reshape(B, H, Sq, N)
    if dtype == "f32":
        assert np.any(np.signbit(d[1][:, :, 300:])) and np.any(~np.signbit(d[1][:, :, 300:]))
