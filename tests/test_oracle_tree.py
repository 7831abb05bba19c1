"""Pins for the oracle's fixed reduction order.

The pages (RL-Kernel PR #453, Summary; RL-Kernel PR #240, Fixed Reduction
Contract) fix a per-tile tree and a left-to-right merge but print no value.
The reading taken is a balanced pairwise tree over key positions; these tests
pin it with (a) a brute-force recursive tree written independently here and
(b) the hand-derived probes in tests/golden/tree_probes.json, whose values
separate the balanced tree from a running sum and from a stride-halving tree.
"""
import json
import os

import numpy as np
import pytest

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tree_probes.json")))


def f32(bits_hex):
    return np.array([int(bits_hex, 16)], np.uint32).view(np.float32)[0]


def bits(x):
    return hex(np.array([x], np.float32).view(np.uint32)[0])


def pairwise_recursive(v):
    """Balanced tree by recursion on halves, float32 adds."""
    v = np.asarray(v, np.float32)
    if v.size == 1:
        return v[0]
    h = v.size // 2
    return np.float32(pairwise_recursive(v[:h]) + pairwise_recursive(v[h:]))


def test_tree_sum_matches_recursive_balanced_tree():
    rng = np.random.default_rng(3)
    differs_from_running = 0
    for trial in range(200):
        # wide dynamic range so that summation order shows in the bits
        v = (rng.standard_normal(256) * np.exp2(rng.integers(-30, 10, 256))).astype(np.float32)
        want = pairwise_recursive(v)
        got = O.tree_sum256(v)
        assert got.tobytes() == want.tobytes(), trial
        run = np.float32(0)
        for a in v:
            run = np.float32(run + a)
        differs_from_running += int(run != got)
    assert differs_from_running > 50


def _bwd_probe_arrays():
    g = GOLD["bwd_probe"]
    N = g["N"]
    vals = {"1": 1.0, "2^-8": 2.0 ** -8, "3*2^-9": 3 * 2.0 ** -9, "2^-9": 2.0 ** -9, "2^-15": 2.0 ** -15}
    P = np.zeros(N, np.float32)
    dP = np.zeros(N, np.float32)
    for k, s in g["P"].items():
        P[int(k)] = vals[s]
    for k, s in g["dP"].items():
        dP[int(k)] = vals[s]
    return P, dP


def test_bwd_probe_delta_is_balanced_tree():
    P, dP = _bwd_probe_arrays()
    g = GOLD["bwd_probe"]
    delta = f32(g["delta_balanced"]["bits"])
    assert delta != f32(g["delta_sequential"]["bits"])
    assert delta != f32(g["delta_stride_halving"]["bits"])
    dS, v = O.bwd(P.reshape(1, 1, 1, -1), dP.reshape(1, 1, 1, -1), 1, 1, 1, 256,
                  p_sink=np.ones(1, np.float32))
    dS = dS.reshape(-1)
    assert bits(dS[0]) == g["dS0"]["bits"]
    assert bits(v[0]) == g["v_with_p_sink_1"]["bits"]
    # every other key: one subtraction and one product with the probe's delta
    want = (P * (dP - delta)).astype(np.float32)
    assert dS.tobytes() == want.tobytes()


def test_bwd_probe_bf16():
    P, dP = _bwd_probe_arrays()
    g = GOLD["bwd_probe"]
    # every probe value is exact in bf16
    Pb = (P.view(np.uint32) >> 16).astype(np.uint16)
    gb = (dP.view(np.uint32) >> 16).astype(np.uint16)
    dS, v = O.bwd(Pb.reshape(1, 1, 1, -1), gb.reshape(1, 1, 1, -1), 1, 1, 1, 256,
                  p_sink=np.ones(1, np.float32))
    # -3*2^-23 is exact in bf16 (0xb4c0)
    assert dS.reshape(-1)[0] == 0xB4C0
    assert bits(v[0]) == g["v_with_p_sink_1"]["bits"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_probe_tile_tree(dtype):
    g = GOLD["fwd_probe"]
    d24 = f32(GOLD["constants"]["d24"]["bits"])
    d32 = f32(GOLD["constants"]["d32"]["bits"])
    assert O.exp_(d24) == np.float32(2.0 ** -24) and O.exp_(d32) == np.float32(2.0 ** -32)
    x = np.full(256, -np.inf, np.float32)
    x[0] = 0.0
    x[2] = x[3] = d24
    if dtype == "f32":
        s, mask = x.reshape(1, 1, 1, -1), None
    else:
        s = np.zeros((1, 1, 1, 256), np.uint16)
        mask = x.copy()
    P, ps = O.fwd(s, 1, 1, 1, 256, mask=mask, mask_strides=(0, 0, 0))
    P = P.reshape(-1)
    if dtype == "f32":
        assert bits(P[0]) == g["P0_f32"]["bits"]
        assert bits(P[2]) == g["P2_f32"]["bits"] and bits(P[3]) == g["P2_f32"]["bits"]
        assert np.all(P[[1] + list(range(4, 256))] == 0)
    else:
        assert P[0] == int(g["P0_bf16"]["bits"], 16)
        assert P[2] == int(g["P2_bf16"]["bits"], 16)
    # with the d32 sink the sink probability shows invL in binary32
    P2, ps2 = O.fwd(s, 1, 1, 1, 256, mask=mask, sink=np.array([d32], np.float32))
    assert bits(ps2[0]) == g["with_sink_d32"]["p_sink"]["bits"]
    assert P2.tobytes() == P.reshape(P2.shape).tobytes()


def test_fold_probe_left_to_right():
    g = GOLD["fold_probe"]
    d24 = f32(GOLD["constants"]["d24"]["bits"])
    x = np.full(513, -np.inf, np.float32)
    x[0] = 0.0
    x[256] = d24
    x[512] = d24
    P, _ = O.fwd(x.reshape(1, 1, 1, -1), 1, 1, 1, 513)
    P = P.reshape(-1)
    assert bits(P[0]) == g["P0_f32"]["bits"]
    assert bits(P[256]) == g["P256_f32"]["bits"]
    assert bits(P[512]) == g["P512_f32"]["bits"]


def test_dsink_probe_chunks_and_fold():
    g = GOLD["dsink_probe"]
    n = g["rows_per_head"]
    v = np.zeros(n, np.float32)
    v[0] = 1.0
    v[256] = v[512] = 2.0 ** -24
    assert bits(O.dsink(v, 1, 1, n)[0]) == g["d_sink"]["bits"]
    w = np.zeros(n, np.float32)
    w[0], w[104], w[193], w[212] = 1.0, 2.0 ** -23, 3 * 2.0 ** -24, 2.0 ** -24
    assert bits(O.dsink(w, 1, 1, n)[0]) == "0x3f800003"
