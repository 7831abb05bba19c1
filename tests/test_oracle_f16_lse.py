"""Pins for the oracle's fp16 dtype and its row log-sum-exp output.

RL-Kernel PR #240 (Path Status: FP16 and BF16 dtypes; Fixed Reduction
Contract, Softmax and LSE: the row's log-sum-exp beside the probabilities).
The binary16 conversions are checked against numpy's own float16 conversion
(round to nearest, ties to even) over every binary16 pattern and a sweep of
binary32 patterns; the fp16 forward and backward must be the fp32 results
rounded once by numpy, and both must agree with float64 softmax; the
log-sum-exp is checked against float64 log-sum-exp and closed forms.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as O
from tests.ref64 import softmax64


def test_f16_decode_every_pattern():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = O.f16_decode(h)
    want = h.view(np.float16).astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("lo", [0x00, 0x01, 0x80])
def test_f16_rne_binary32_sweep(lo):
    # 2^24 binary32 patterns per case: every sign, exponent and top 15
    # fraction bits (which decide binary16 ties and their sticky bits), with
    # the low byte fixed
    u = ((np.arange(1 << 24, dtype=np.uint32) << np.uint32(8)) | np.uint32(lo))
    x = u.view(np.float32)
    got = O.f16_rne(x)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    g = got[nan]
    assert np.all((g & 0x7c00) == 0x7c00) and np.all((g & 0x3ff) != 0)


def test_f16_rne_edges():
    vals = np.array([65504, 65519.99, 65520, 65536, 1e30, np.inf, -np.inf, 2.0 ** -14,
                     2.0 ** -24, 2.0 ** -25, np.nextafter(np.float32(2.0 ** -25), 1),
                     3 * 2.0 ** -26, 2.0 ** -15 * (1 + 2.0 ** -11), 0.0, -0.0, 1.0 + 2.0 ** -11,
                     1.0 + 3 * 2.0 ** -11, 1e-45], np.float32)
    got = O.f16_rne(vals)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def _rand_rows(seed, shape, std):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * std).astype(np.float16)


@pytest.mark.parametrize("N", [1, 7, 256, 257, 700, 4352])
def test_f16_forward_is_fp32_forward_rounded_once(N):
    B, H, Sq = 2, 2, 5
    s16 = _rand_rows(N, (B, H, Sq, N), 3.0)
    s32 = s16.astype(np.float32)
    sink = np.array([0.5, -1.0], np.float32)
    mask = np.zeros((B, N), np.float32)
    mask[1, N // 2:] = -np.inf
    P16, ps16, l16 = O.fwd(s16, B, H, Sq, N, mask=mask, mask_strides=(N, 0, 0), sink=sink,
                           want_lse=True)
    P32, ps32, l32 = O.fwd(s32, B, H, Sq, N, mask=mask, mask_strides=(N, 0, 0), sink=sink,
                           want_lse=True)
    assert P16.dtype == np.float16
    assert np.array_equal(P16.view(np.uint16), P32.astype(np.float16).view(np.uint16))
    assert ps16.tobytes() == ps32.tobytes() and l16.tobytes() == l32.tobytes()
    # and against float64 softmax: one binary16 rounding (2^-11 relative for
    # normal results, half of 2^-24 absolute below 2^-14) on top of fp32 error
    x = s32.reshape(B * H, Sq, N).astype(np.float64)
    for r in range(B * H):
        b, h = divmod(r, H)
        Pref, _ = softmax64(x[r] + mask[b], np.full(Sq, float(sink[h])))
        got = P16.reshape(B * H, Sq, N)[r].astype(np.float64)
        assert np.all(np.abs(got - Pref) <= 2.0 ** -11 * Pref * 1.01 + 2.0 ** -25 + 1e-12)


@pytest.mark.parametrize("N", [257, 4352])
def test_f16_backward_is_fp32_backward_rounded_once(N):
    B, H, Sq = 1, 3, 6
    rng = np.random.default_rng(N + 1)
    P16 = (np.abs(rng.standard_normal((B, H, Sq, N))) * (2.0 / N)).astype(np.float16)
    g16 = rng.standard_normal((B, H, Sq, N)).astype(np.float16)
    ps = rng.random(B * H * Sq).astype(np.float32)
    dS16, v16 = O.bwd(P16, g16, B, H, Sq, N, p_sink=ps)
    dS32, v32 = O.bwd(P16.astype(np.float32), g16.astype(np.float32), B, H, Sq, N, p_sink=ps)
    assert np.array_equal(dS16.view(np.uint16), dS32.astype(np.float16).view(np.uint16))
    assert v16.tobytes() == v32.tobytes()
    # float64 VJP: dS = P (dP - sum P dP)
    p = P16.astype(np.float64).reshape(-1, N)
    g = g16.astype(np.float64).reshape(-1, N)
    d64 = p * (g - (p * g).sum(axis=1, keepdims=True))
    got = dS16.astype(np.float64).reshape(-1, N)
    scale = p * (np.abs(g) + np.abs((p * g).sum(axis=1, keepdims=True)))
    assert np.all(np.abs(got - d64) <= 2.0 ** -11 * np.abs(d64) + 1e-5 * scale + 2.0 ** -25)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_lse_against_float64(dtype):
    B, H, Sq, N = 2, 2, 9, 1000
    rng = np.random.default_rng(3)
    s32 = (rng.standard_normal((B, H, Sq, N)) * 4).astype(np.float32)
    if dtype == "f16":
        s = s32.astype(np.float16)
        x = s.astype(np.float64)
    elif dtype == "bf16":
        from tests.ref64 import f32_to_bf16_bits_torch
        s = f32_to_bf16_bits_torch(s32)
        x = (s.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    else:
        s = s32
        x = s32.astype(np.float64)
    sink = np.array([1.5, -0.25], np.float32)
    _, _, lse = O.fwd(s, B, H, Sq, N, sink=sink, causal=True, want_lse=True)
    xr = x.reshape(B * H, Sq, N)
    vis = np.arange(N)[None, :] <= (N - Sq) + np.arange(Sq)[:, None]
    for r in range(B * H):
        h = r % H
        z = np.where(vis, xr[r], -np.inf)
        want = logsumexp(np.concatenate([z, np.full((Sq, 1), float(sink[h]))], axis=1), axis=1)
        got = lse.reshape(B * H, Sq)[r].astype(np.float64)
        assert np.all(np.abs(got - want) <= 4e-6 * np.maximum(1.0, np.abs(want)))


def test_lse_closed_forms():
    N = 700
    # N equal scores c: c + ln N
    for c in (0.0, 3.0, -20.0):
        s = np.full((1, 1, 1, N), c, np.float32)
        _, _, lse = O.fwd(s, 1, 1, 1, N, want_lse=True)
        assert abs(float(lse[0]) - (c + math.log(N))) <= 4e-6 * max(1.0, abs(c + math.log(N)))
    # one visible key: its score exactly (L = 1, ln 1 = 0)
    s = np.full((1, 1, 1, N), 2.5, np.float32)
    s[0, 0, 0, 0] = 1.25
    _, _, lse = O.fwd(s, 1, 1, 1, N, key_len=np.array([1], np.int32), want_lse=True)
    assert lse[0] == np.float32(1.25)
    # nothing visible: -inf; with a sink, the sink logit exactly
    _, _, lse = O.fwd(s, 1, 1, 1, N, key_len=np.array([0], np.int32), want_lse=True)
    assert lse[0] == -np.inf
    _, ps, lse = O.fwd(s, 1, 1, 1, N, key_len=np.array([0], np.int32),
                       sink=np.array([-0.75], np.float32), want_lse=True)
    assert lse[0] == np.float32(-0.75) and ps[0] == 1.0


def test_probabilities_are_exp_of_score_minus_lse():
    B, H, Sq, N = 1, 1, 4, 513
    s = (np.random.default_rng(9).standard_normal((B, H, Sq, N)) * 2).astype(np.float32)
    P, _, lse = O.fwd(s, B, H, Sq, N, want_lse=True)
    want = np.exp(s.reshape(Sq, N).astype(np.float64) - lse.astype(np.float64)[:, None])
    assert np.allclose(P.reshape(Sq, N), want, rtol=1e-5, atol=1e-30)
