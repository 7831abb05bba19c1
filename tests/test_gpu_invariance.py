"""GPU batch invariance and edge cases.

RL-Kernel PR #453 (Summary): a row must not change with its batch, launch
geometry or backend.  RL-Kernel PR #240 (Acceptance Criteria): batch size and
batch position invariance are bitwise for the same physical row shape.  Here:
the fp32 8,449-key sweep over batches of 1, 3, 17, 64 (x 32 heads) with a
fixed block of rows at a random position, every compiled launch geometry, the
element-wise and 16-byte paths, in-place calls and run-to-run repeats, all
compared byte for byte; plus the degenerate cases the method has.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import oracle
import synth
from tests.gpu_util import assert_bitexact, assert_close, dev, log

pytestmark = pytest.mark.gpu
GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "tree_probes.json")))


def bits(t):
    return synth.to_numpy_bits(t)


def test_batch_invariance_fp32_8449_keys():
    H, N = 32, 8449
    ref = None
    for n in (1, 3, 17, 64):
        log(f"batch sweep: fp32 [{n},{H},1,{N}] fwd+bwd")
        s, g, p = synth.batch_sweep_fp32(n, device="cpu")
        P, _ = jas.fwd(s.to(dev()))
        dS, _ = jas.bwd(P, g.to(dev()))
        torch.cuda.synchronize()
        blk = (bits(P[p]), bits(dS[p]))
        if ref is None:
            ref = blk
            # the fixed block against the oracle (forward), and the backward
            # stage-isolated on the oracle's P
            s_np = bits(s[p:p + 1])
            P_o, _ = oracle.fwd(s_np, 1, H, 1, N)
            assert_close(blk[0].reshape(P_o.shape), P_o, "batch sweep P")
            Pin = synth.from_numpy_bits(P_o, dev())
            dSi, _ = jas.bwd(Pin, g[p:p + 1].to(dev()))
            torch.cuda.synchronize()
            dS_o, _ = oracle.bwd(P_o, bits(g[p:p + 1]), 1, H, 1, N)
            assert_bitexact(bits(dSi), dS_o, "batch sweep dS")
        else:
            assert blk[0].tobytes() == ref[0].tobytes(), f"P bytes changed at batch {n}"
            assert blk[1].tobytes() == ref[1].tobytes(), f"dS bytes changed at batch {n}"


def valid_geometries(dtype, N):
    tps = 1 if dtype == torch.float32 else 2
    T = (N + 255) // 256
    nslots = (T + tps - 1) // tps
    cpls = [1, 2, 3, 5, 9] + ([17] if dtype == torch.float32 else [])
    out = []
    for w in (1, 2, 4):
        for c in cpls:
            if w * c >= nslots:
                for rpb in range(1, 4 // w + 1):
                    out.append((w, c, rpb, 0))
    out.append((out[0][0], out[0][1], out[0][2], 3))  # grid of 3 workgroups looping over rows
    return out


@pytest.mark.parametrize("dt,N", [(torch.bfloat16, 4352), (torch.float32, 8449),
                                  (torch.bfloat16, 700), (torch.float32, 257),
                                  (torch.bfloat16, 16384), (torch.float16, 4352),
                                  (torch.float16, 700)])
def test_every_launch_geometry_gives_identical_bytes(dt, N):
    B, H, S = 1, 3, 5
    s = synth.normal((B, H, S, N), 2.0, 200 + N, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 201 + N, "cpu", dt).to(dev())
    mask = torch.zeros((B, 1, 1, N), device=dev())
    mask[..., N - 37:] = float("-inf")
    sink = synth.normal((H,), 1.0, 202 + N, "cpu").to(dev())
    geos = valid_geometries(dt, N)
    log(f"geometries: {dt} N={N}: {len(geos)}")
    ref = None
    for L in geos:
        P, ps, lse = jas.fwd(s, mask=mask, sink=sink, launch=L, want_lse=True)
        dS, dsk = jas.bwd(P, g, p_sink=ps, launch=L)
        torch.cuda.synchronize()
        cur = (bits(P).tobytes(), ps.cpu().numpy().tobytes(), bits(dS).tobytes(),
               dsk.cpu().numpy().tobytes(), lse.cpu().numpy().tobytes())
        if ref is None:
            ref = cur
        else:
            assert cur == ref, f"launch {L} changed the bytes"


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_elementwise_path_matches_vector_path(dt):
    # a row stride with padding that breaks 16-byte alignment, and a base
    # offset by one element, take the element-wise path; bytes must not move
    B, H, S, N = 1, 2, 7, 4352
    s = synth.normal((B, H, S, N), 2.0, 300, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 301, "cpu", dt).to(dev())
    sink = synth.normal((H,), 1.0, 302, "cpu").to(dev())
    P0, ps0 = jas.fwd(s, sink=sink)
    dS0, d0 = jas.bwd(P0, g, p_sink=ps0)
    for pad, off in ((3, 0), (0, 1), (5, 1)):
        ld = N + pad
        big = torch.zeros(B * H * S * ld + off, dtype=dt, device=dev())
        sv = big[off:].view(B, H, S, ld)[..., :N]
        sv.copy_(s)
        gbig = torch.zeros_like(big)
        gv = gbig[off:].view(B, H, S, ld)[..., :N]
        gv.copy_(g)
        P1, ps1 = jas.fwd(sv, sink=sink)          # out: same row stride
        assert P1.stride() == sv.stride()
        Pbig = torch.full_like(big, 7.0)
        Pv = Pbig[off:].view(B, H, S, ld)[..., :N]
        jas.fwd(sv, sink=sink, out=Pv, p_sink=torch.empty_like(ps0))
        dbig = torch.full_like(big, 5.0)
        dv = dbig[off:].view(B, H, S, ld)[..., :N]
        _, d1 = jas.bwd(Pv, gv, p_sink=ps0, out=dv)
        torch.cuda.synchronize()
        assert bits(P1).tobytes() == bits(P0).tobytes()
        assert bits(Pv.contiguous()).tobytes() == bits(P0).tobytes()
        assert bits(dv.contiguous()).tobytes() == bits(dS0).tobytes()
        assert d1.cpu().numpy().tobytes() == d0.cpu().numpy().tobytes()
        # the padding between rows is never written
        if pad:
            pad_vals = Pbig[off:].view(B, H, S, ld)[..., N:]
            assert torch.all(pad_vals == 7.0)


def test_in_place_and_repeat():
    B, H, S, N = 2, 2, 9, 4352
    s = synth.normal((B, H, S, N), 2.0, 400, "cpu", torch.bfloat16).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 401, "cpu", torch.bfloat16).to(dev())
    P0, _ = jas.fwd(s)
    dS0, _ = jas.bwd(P0, g)
    P1, _ = jas.fwd(s)
    x = s.clone()
    jas.fwd(x, out=x)                               # probs == scores
    y = g.clone()
    Pc = P0.clone()
    jas.bwd(Pc, y, out=y)                           # dscores == dprobs
    z = P0.clone()
    jas.bwd(z, g, out=z)                            # dscores == probs
    torch.cuda.synchronize()
    assert torch.equal(bits_t(P0), bits_t(P1))
    assert torch.equal(bits_t(x), bits_t(P0))
    assert torch.equal(bits_t(y), bits_t(dS0))
    assert torch.equal(bits_t(z), bits_t(dS0))


def bits_t(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def test_one_head_sliced_from_the_batch():
    # one head's rows taken as a call of their own through a slice of the
    # batch (torch leaves the size-1 batch and head dimensions' strides at
    # the parent's values): the same bytes as in the whole call, with the
    # mask, the sink, the causal cut, the lse and d_sink
    B, H, S, N = 1, 5, 33, 1000
    s = synth.normal((B, H, S, N), 2.0, 410, "cpu", torch.bfloat16).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 411, "cpu", torch.bfloat16).to(dev())
    mask = torch.zeros((B, 1, 1, N), device=dev())
    mask[..., 900:] = float("-inf")
    sink = synth.normal((H,), 1.0, 412, "cpu").to(dev())
    P, ps, lse = jas.fwd(s, mask=mask, sink=sink, causal=True, want_lse=True)
    dS, dsk = jas.bwd(P, g, p_sink=ps, causal=True)
    for h in (0, 3):
        sh, gh = s[:, h:h + 1], g[:, h:h + 1]
        assert sh.stride(0) != sh.shape[1] * sh.stride(1)   # the parent's batch stride
        Ph, psh, lseh = jas.fwd(sh, mask=mask, sink=sink[h:h + 1], causal=True, want_lse=True)
        dSh, dskh = jas.bwd(Ph, gh, p_sink=psh, causal=True)
        torch.cuda.synchronize()
        rows = slice(h * S, (h + 1) * S)
        assert torch.equal(bits_t(Ph), bits_t(P[:, h:h + 1]))
        assert torch.equal(bits_t(psh), bits_t(ps[rows])) and torch.equal(bits_t(lseh), bits_t(lse[rows]))
        assert torch.equal(bits_t(dSh), bits_t(dS[:, h:h + 1]))
        assert torch.equal(bits_t(dskh), bits_t(dsk[h:h + 1]))


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_degenerate_rows(dt):
    N = 600
    rows = 6
    s = torch.zeros((1, 1, rows, N), dtype=torch.float32)
    s[0, 0, 0, :] = 0.375                               # uniform -> fl(1/N)
    s[0, 0, 1, :] = float("-inf")                       # one-hot
    s[0, 0, 1, 437] = -12.25
    s[0, 0, 2, :] = float("-inf")                       # all -inf
    s[0, 0, 3, :] = torch.linspace(-3, 3, N)
    s[0, 0, 4, :] = 0.375
    s[0, 0, 5, :] = torch.arange(N) % 7 - 3.0
    sd = s.to(dt).to(dev())
    P, _, lse = jas.fwd(sd, want_lse=True)
    Pn, psn, lsen = jas.fwd(sd, sink=torch.full((1,), float("-inf"), device=dev()),
                            want_lse=True)
    torch.cuda.synchronize()
    # log-sum-exp closed forms: one finite key gives its score exactly (L = 1),
    # nothing finite gives -inf, a uniform row c + ln N within the tolerance
    lc = lse.cpu()
    assert lc[1].item() == -12.25 and lc[2].item() == float("-inf")
    assert abs(lc[0].item() - (0.375 + math.log(N))) <= 4e-6 * (0.375 + math.log(N))
    assert torch.equal(bits_t(lse), bits_t(lsen))
    Pf = P.float().cpu()
    if dt == torch.float32:
        assert torch.all(Pf[0, 0, 0] == torch.tensor(1.0, dtype=torch.float32) / N)
    assert Pf[0, 0, 1, 437] == 1.0 and torch.count_nonzero(Pf[0, 0, 1]) == 1
    assert torch.all(Pf[0, 0, 2] == 0) and not torch.any(torch.signbit(Pf[0, 0, 2]))
    # a -inf sink is the same as no sink, with p_sink = 0
    assert torch.equal(bits_t(P), bits_t(Pn)) and torch.all(psn == 0)
    # fully masked row with a sink: P = 0, p_sink = 1
    P2, ps2, lse2 = jas.fwd(sd, sink=torch.zeros(1, device=dev()), want_lse=True)
    torch.cuda.synchronize()
    assert torch.all(P2[0, 0, 2] == 0) and ps2[2].item() == 1.0 and lse2[2].item() == 0.0
    # uniform row with sink equal to the row value: P = p_sink = fl(1/(N+1))
    P3, ps3 = jas.fwd(sd, sink=torch.full((1,), 0.375, device=dev()))
    torch.cuda.synchronize()
    want = (torch.tensor(1.0, dtype=torch.float32) / (N + 1)).item()
    assert ps3[0].item() == want
    if dt == torch.float32:
        assert torch.all(P3[0, 0, 0].cpu() == want)
    # single key
    P1k, _ = jas.fwd(torch.tensor([[[[3.5]]]], dtype=dt, device=dev()))
    torch.cuda.synchronize()
    assert P1k.item() == 1.0


def test_tree_and_fold_probes_on_gpu():
    # the hand-derived probes of tests/golden/tree_probes.json, bitwise
    gb, gf, gd = GOLD["bwd_probe"], GOLD["fwd_probe"], GOLD["fold_probe"]

    def f32(h):
        return np.array([int(h, 16)], np.uint32).view(np.float32)[0]

    d24 = f32(GOLD["constants"]["d24"]["bits"])
    d32 = f32(GOLD["constants"]["d32"]["bits"])
    # backward probe, fp32 and bf16
    vals = {"1": 1.0, "2^-8": 2.0 ** -8, "3*2^-9": 3 * 2.0 ** -9, "2^-9": 2.0 ** -9, "2^-15": 2.0 ** -15}
    P = torch.zeros(256)
    G = torch.zeros(256)
    for k, v in gb["P"].items():
        P[int(k)] = vals[v]
    for k, v in gb["dP"].items():
        G[int(k)] = vals[v]
    for dt in (torch.float32, torch.bfloat16):
        dS, dsk = jas.bwd(P.to(dt).view(1, 1, 1, 256).to(dev()), G.to(dt).view(1, 1, 1, 256).to(dev()),
                          p_sink=torch.ones(1, device=dev()))
        torch.cuda.synchronize()
        assert dS[0, 0, 0, 0].float().item() == float(f32(gb["dS0"]["bits"]))
        assert dsk.cpu().numpy().view(np.uint32)[0] == int(gb["v_with_p_sink_1"]["bits"], 16)
    # forward probe (fp32 scores; bf16 scores with the values in the mask)
    x = torch.full((256,), float("-inf"))
    x[0] = 0.0
    x[2] = x[3] = float(d24)
    P, ps = jas.fwd(x.view(1, 1, 1, 256).to(dev()), sink=torch.tensor([float(d32)], device=dev()))
    Pb, psb = jas.fwd(torch.zeros((1, 1, 1, 256), dtype=torch.bfloat16, device=dev()),
                      mask=x.view(1, 1, 1, 256).to(dev()),
                      sink=torch.tensor([float(d32)], device=dev()))
    torch.cuda.synchronize()
    pv = P.cpu().numpy().reshape(-1).view(np.uint32)
    assert pv[0] == int(gf["P0_f32"]["bits"], 16) and pv[2] == int(gf["P2_f32"]["bits"], 16)
    assert ps.cpu().numpy().view(np.uint32)[0] == int(gf["with_sink_d32"]["p_sink"]["bits"], 16)
    pb = bits(Pb).reshape(-1)
    assert pb[0] == int(gf["P0_bf16"]["bits"], 16) and pb[2] == int(gf["P2_bf16"]["bits"], 16)
    assert psb.cpu().numpy().view(np.uint32)[0] == int(gf["with_sink_d32"]["p_sink"]["bits"], 16)
    # fold probe: three tiles, the last of one key
    x = torch.full((513,), float("-inf"))
    x[0] = 0.0
    x[256] = float(d24)
    x[512] = float(d24)
    P, _ = jas.fwd(x.view(1, 1, 1, 513).to(dev()))
    torch.cuda.synchronize()
    pv = P.cpu().numpy().reshape(-1).view(np.uint32)
    assert pv[0] == int(gd["P0_f32"]["bits"], 16)
    assert pv[256] == int(gd["P256_f32"]["bits"], 16) and pv[512] == int(gd["P512_f32"]["bits"], 16)


def test_dsink_chunk_probe_on_gpu():
    # rows of one head carrying p_sink*delta = the d_sink probe's values:
    # P = one-hot (key 0), dP = -v at key 0, p_sink = 1 -> share = -(1*delta) = v
    g = GOLD["dsink_probe"]
    n = g["rows_per_head"]
    v = torch.zeros(n)
    v[0] = 1.0
    v[256] = v[512] = 2.0 ** -24
    P = torch.zeros((1, 1, n, 8))
    P[..., 0] = 1.0
    G = torch.zeros((1, 1, n, 8))
    G[0, 0, :, 0] = -v
    _, dsk = jas.bwd(P.to(dev()), G.to(dev()), p_sink=torch.ones(n, device=dev()))
    torch.cuda.synchronize()
    assert dsk.cpu().numpy().view(np.uint32)[0] == int(g["d_sink"]["bits"], 16)


def test_empty_calls():
    e = torch.empty((0, 3, 5, 300), dtype=torch.bfloat16, device=dev())
    P, ps = jas.fwd(e, sink=torch.zeros(3, device=dev()))
    d = torch.full((3,), 9.0, device=dev())
    dS, dsk = jas.bwd(P, e, p_sink=ps, d_sink=d)
    torch.cuda.synchronize()
    assert P.numel() == 0 and torch.all(dsk == 0) and not torch.any(torch.signbit(dsk))
