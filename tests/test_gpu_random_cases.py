"""GPU: seeded random configurations against the oracle, to reach the
combinations the hand-picked cases do not.

Each softmax case draws a dtype, a shape (1 to 40,000 keys: one-pass and
streaming rows, tails of every size), padded rows (ld > N, which also moves
rows off 16-byte boundaries), a mask with broadcast or per-query strides and
-inf entries, the sink, the causal flag and key lengths (including 0, past
the row and negative), and checks every row: the forward within 1 ulp of
the dtype (4e-6 relative for fp32) with the row log-sum-exp (and, for
16-bit rows of 2 to 10 slots with a mask, byte-identical with the mask kept
in registers on a random grid), and the
backward stage-isolated (the oracle's P and p_sink, a synthetic dP) bit for
bit, d_sink included.  RL-Kernel PR #453, Summary and Fixed-order backward;
ROCm TransformerEngine PR #678 (sink); RL-Kernel PR #240, Path Status
(causal and padding masks).

Each attention case draws a dtype, head dim, grouped heads, shape, mask,
sink, causal flag and key lengths and applies the fused attention checks of
test_gpu_attention.
"""
import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import oracle
import synth
from tests.gpu_util import assert_bitexact, assert_close, assert_lse_close, dev, log
from tests.test_gpu_attention import check as attn_check, draw as attn_draw

pytestmark = pytest.mark.gpu

DTYPES = [torch.float32, torch.bfloat16, torch.float16]


def draw_case(i):
    rng = np.random.default_rng(7000 + i)
    dt = DTYPES[rng.integers(3)]
    u = rng.random()
    N = int(rng.integers(1, 40) if u < 0.1 else rng.integers(40, 600) if u < 0.45
            else rng.integers(600, 5000) if u < 0.72 else rng.integers(5000, 16385) if u < 0.86
            else rng.integers(16385, 40001))
    budget = 2_500_000 // N
    B = int(rng.integers(1, 4))
    H = int(rng.integers(1, 5))
    Sq = int(max(1, min(rng.integers(1, 41), budget // (B * H))))
    pad = int(rng.choice([0, 0, rng.integers(1, 10)]))
    mask_kind = rng.choice(["none", "batch", "query"])
    return dict(dt=dt, B=B, H=H, Sq=Sq, N=N, pad=pad, mask_kind=str(mask_kind),
                sink=bool(rng.random() < 0.5), causal=bool(rng.random() < 0.3),
                key_len=bool(rng.random() < 0.3), seed=int(7000 + i), rng=rng)


@pytest.mark.parametrize("i", range(60))
def test_random_softmax_case(i):
    c = draw_case(i)
    dt, B, H, Sq, N, pad, rng = c["dt"], c["B"], c["H"], c["Sq"], c["N"], c["pad"], c["rng"]
    ld = N + pad
    rows = B * H * Sq
    log(f"case {i}: {dt} B={B} H={H} Sq={Sq} N={N} ld={ld} mask={c['mask_kind']} "
        f"sink={c['sink']} causal={c['causal']} key_len={c['key_len']}")
    full = synth.normal((B, H, Sq, ld), 3.0, c["seed"], "cpu", dt)
    s_bits = synth.to_numpy_bits(full)
    s = synth.from_numpy_bits(s_bits, dev())[..., :N]            # rows of stride ld on the GPU
    mask = ms = None
    if c["mask_kind"] == "batch":
        mask = synth.normal((B, N), 1.0, c["seed"] + 1, "cpu")
        mask[torch.rand((B, N), generator=torch.Generator().manual_seed(c["seed"])) < 0.05] = float("-inf")
        ms = (N, 0, 0)
    elif c["mask_kind"] == "query":
        mq = N + int(rng.integers(0, 4))                          # rows not always 16-byte aligned
        mask = synth.normal((B * H * Sq * mq,), 1.0, c["seed"] + 1, "cpu")
        mask[:: int(rng.integers(3, 30))] = float("-inf")
        ms = (H * Sq * mq, Sq * mq, mq)
    sink = synth.normal((H,), 1.5, c["seed"] + 2, "cpu") if c["sink"] else None
    kl = None
    if c["key_len"]:
        kl = np.array([int(rng.integers(-3, N + 6)) if rng.random() < 0.8 else N for _ in range(B)],
                      np.int32)
    kw = dict(causal=c["causal"], key_len=None if kl is None else torch.from_numpy(kl).to(dev()))
    P, ps, lse = jas.fwd(s, mask=None if mask is None else mask.to(dev()), mask_strides=ms,
                         sink=None if sink is None else sink.to(dev()), want_lse=True, **kw)
    torch.cuda.synchronize()
    P_o, ps_o, lse_o = oracle.fwd(s_bits, B, H, Sq, N, ld=ld,
                                  mask=None if mask is None else mask.numpy(),
                                  mask_strides=ms or (0, 0, 0),
                                  sink=None if sink is None else sink.numpy(), causal=c["causal"],
                                  key_len=kl, want_lse=True)
    got = synth.to_numpy_bits(P.contiguous()).reshape(rows, N)
    want = P_o.reshape(rows, ld)[:, :N]
    assert_close(got, np.ascontiguousarray(want), f"case {i} P")
    assert_lse_close(lse.cpu().numpy(), lse_o, f"case {i} lse")
    if sink is not None:
        assert_close(ps.cpu().numpy(), ps_o, f"case {i} p_sink")
    # where it is built (16-bit rows of 2 to 10 slots with a mask), the
    # forward with the mask kept in registers gives the same bytes
    if mask is not None and dt != torch.float32 and 512 < N <= 5120:
        grid = int(rng.integers(1, rows + 1))
        P2, ps2, lse2 = jas.fwd(s, mask=mask.to(dev()), mask_strides=ms,
                                sink=None if sink is None else sink.to(dev()), want_lse=True,
                                launch=(0, 0, 0, grid, 0, 1), **kw)
        torch.cuda.synchronize()
        assert torch.equal(P2, P) and torch.equal(lse2, lse), f"case {i} mask in registers"
        if sink is not None:
            assert torch.equal(ps2, ps)
    # backward, stage-isolated: the oracle's P and p_sink, a synthetic dP
    g_full = synth.normal((B, H, Sq, ld), 1.0, c["seed"] + 3, "cpu", dt)
    g_bits = synth.to_numpy_bits(g_full)
    Pin = synth.from_numpy_bits(P_o.reshape(B, H, Sq, ld), dev())[..., :N]
    gin = synth.from_numpy_bits(g_bits, dev())[..., :N]
    psin = None if ps_o is None else torch.from_numpy(ps_o).to(dev())
    dS, dsk = jas.bwd(Pin, gin, p_sink=psin, **kw)
    torch.cuda.synchronize()
    dS_o, v_o = oracle.bwd(P_o, g_bits, B, H, Sq, N, ld=ld, p_sink=ps_o, causal=c["causal"],
                           key_len=kl)
    assert_bitexact(synth.to_numpy_bits(dS.contiguous()).reshape(rows, N),
                    np.ascontiguousarray(dS_o.reshape(rows, ld)[:, :N]), f"case {i} dS")
    if sink is not None:
        assert_bitexact(dsk.cpu().numpy(), oracle.dsink(v_o, B, H, Sq), f"case {i} d_sink")


@pytest.mark.parametrize("i", range(32))
def test_random_attention_case(i):
    rng = np.random.default_rng(9000 + i)
    dt = [torch.bfloat16, torch.float16][rng.integers(2)]
    D = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.integers(1, 4))
    B = int(rng.integers(1, 3))
    N = int(rng.integers(1, 2500))
    Sq = int(rng.integers(1, 150))
    log(f"attention case {i}: {dt} D={D} B={B} H={H} Hkv={Hkv} Sq={Sq} N={N}")
    q, k, v = attn_draw(9000 + i, B, H, Hkv, Sq, N, D, dt, std=float(rng.uniform(0.5, 1.5)))
    mask = ms = None
    if rng.random() < 0.5:
        mq = N + int(rng.integers(0, 3))
        mask = synth.normal((B * H * Sq * mq,), 1.0, 9100 + i, "cpu")
        mask[:: int(rng.integers(4, 40))] = float("-inf")
        ms = (H * Sq * mq, Sq * mq, mq)
    sink = synth.normal((H,), 1.0, 9200 + i, "cpu") if rng.random() < 0.5 else None
    kl = [int(rng.integers(-2, N + 4)) for _ in range(B)] if rng.random() < 0.4 else None
    attn_check(q, k, v, float(rng.uniform(0.05, 0.2)), mask=mask, mask_strides=ms, sink=sink,
               causal=bool(rng.random() < 0.4), kl=kl)
