"""GPU: the streaming kernels, for rows longer than the one-pass kernels hold
(more than 16,384 keys, up to 262,144).

RL-Kernel PR #453, Summary: the row is processed tile by tile, left to
right, the per-tile states merged in order; nothing in the result depends on
how many tiles are held at once.  So the streaming kernels, forced onto rows
the one-pass kernels also run, must give the same bytes (P, p_sink, lse, dS,
d_sink), and on long rows they are checked against the oracle: forward to
the usual tolerance, backward stage-isolated and bit-exact.
"""
import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import oracle
import synth
from tests.gpu_util import (assert_bitexact, assert_close, assert_lse_close, dev, gather_rows,
                            log, oracle_rows_bwd, sample_rows)

pytestmark = pytest.mark.gpu

STREAM_CPLS = {torch.float32: (8, 16), torch.bfloat16: (4, 8), torch.float16: (4, 8)}


def run(s, g, launch=None, mask=None, mask_strides=None, sink=None, causal=False, key_len=None):
    P, ps, lse = jas.fwd(s, mask=mask, mask_strides=mask_strides, sink=sink, causal=causal,
                         key_len=key_len, launch=launch, want_lse=True)
    dS, dsk = jas.bwd(P, g, p_sink=ps, causal=causal, key_len=key_len, launch=launch)
    torch.cuda.synchronize()
    out = [synth.to_numpy_bits(P).tobytes(), lse.cpu().numpy().tobytes(),
           synth.to_numpy_bits(dS).tobytes()]
    if sink is not None:
        out += [ps.cpu().numpy().tobytes(), dsk.cpu().numpy().tobytes()]
    return out


@pytest.mark.parametrize("N", [1, 7, 257, 700, 4352, 8449, 16384])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_forced_streaming_matches_one_pass(dt, N):
    B, H, S = 2, 2, 5
    log(f"forced streaming vs one pass: {dt} N={N}")
    s = synth.normal((B, H, S, N), 2.0, 400 + N, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 401 + N, "cpu", dt).to(dev())
    mask = torch.zeros((B, 1, 1, N), device=dev())
    mask[1, ..., N - N // 3:] = float("-inf")
    sink = synth.normal((H,), 1.0, 402 + N, "cpu").to(dev())
    kl = torch.tensor([N, max(0, N - 300)], dtype=torch.int32, device=dev())
    cases = [dict(), dict(mask=mask, sink=sink), dict(causal=True, sink=sink),
             dict(key_len=kl, mask=mask)]
    for kw in cases:
        ref = run(s, g, **kw)
        for cpl in STREAM_CPLS[dt]:
            got = run(s, g, launch=(4, cpl, 1, 0, 1), **kw)
            assert got == ref, f"streaming cpl={cpl} {sorted(kw)} changed the bytes"
        if dt != torch.float32:  # the 16-wave workgroup (16-bit types)
            got = run(s, g, launch=(8, 8, 1, 0, 1), **kw)
            assert got == ref, f"wide streaming {sorted(kw)} changed the bytes"


def long_case(dt, N, B=1, H=2, S=3, with_mask=False, with_sink=False, causal=False, kl=None,
              seed=0):
    s = synth.normal((B, H, S, N), 2.0, seed, "cpu", dt)
    mask = None
    if with_mask:
        mask = torch.zeros((B, 1, 1, N))
        mask[..., N // 2:N // 2 + 1000] = float("-inf")
    sink = synth.normal((H,), 1.0, seed + 2, "cpu") if with_sink else None
    key_len = None if kl is None else torch.tensor(kl, dtype=torch.int32)
    P, ps, lse = jas.fwd(s.to(dev()), mask=None if mask is None else mask.to(dev()),
                         mask_strides=None if mask is None else (N, 0, 0),
                         sink=None if sink is None else sink.to(dev()), causal=causal,
                         key_len=None if key_len is None else key_len.to(dev()), want_lse=True)
    torch.cuda.synchronize()
    P_o, ps_o, lse_o = oracle.fwd(synth.to_numpy_bits(s), B, H, S, N,
                                  mask=None if mask is None else mask.numpy(),
                                  mask_strides=(N, 0, 0), sink=None if sink is None else sink.numpy(),
                                  causal=causal, key_len=None if kl is None else np.array(kl, np.int32),
                                  want_lse=True)
    assert_close(synth.to_numpy_bits(P), P_o, f"P N={N}")
    assert_lse_close(lse.cpu().numpy(), lse_o, f"lse N={N}")
    if with_sink:
        assert_close(ps.cpu().numpy(), ps_o, "p_sink")
    # stage-isolated backward on the oracle's P
    g = synth.normal((B, H, S, N), 1.0, seed + 1, "cpu", dt)
    Pin = synth.from_numpy_bits(P_o, dev())
    psin = None if ps_o is None else torch.from_numpy(ps_o).to(dev())
    dS, dsk = jas.bwd(Pin, g.to(dev()), p_sink=psin, causal=causal,
                      key_len=None if key_len is None else key_len.to(dev()))
    torch.cuda.synchronize()
    dS_o, v_o = oracle.bwd(P_o, synth.to_numpy_bits(g), B, H, S, N, p_sink=ps_o, causal=causal,
                           key_len=None if kl is None else np.array(kl, np.int32))
    assert_bitexact(synth.to_numpy_bits(dS), dS_o, f"dS N={N}")
    if with_sink:
        assert_bitexact(dsk.cpu().numpy(), oracle.dsink(v_o, B, H, S), "d_sink")


@pytest.mark.parametrize("N", [16385, 20000, 32768, 65536, 100003, 262144])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_long_rows_against_oracle(dt, N):
    log(f"long rows: {dt} N={N}")
    long_case(dt, N, with_mask=N % 2 == 0, with_sink=True, seed=N % 1000)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_near_uniform_long_row_lse(dt):
    # L close to its largest value N + 1: every score within 2^-6 of 0 and a
    # sink of 0, so each of the 262,144 keys adds nearly 1 and the hardware
    # logarithm sees L near 2^18 (the top of its probed range)
    N, B, H, S = 262144, 1, 2, 2
    log(f"near-uniform long rows, lse: {dt} N={N}")
    z = synth.normal((B, H, S, N), 1.0, 610, "cpu")
    s = (torch.round(z * 2.0) * 2.0 ** -8).to(dt)   # multiples of 2^-8 in about [-2^-6, 2^-6]
    sink = torch.zeros(H)
    P, ps, lse = jas.fwd(s.to(dev()), sink=sink.to(dev()), want_lse=True)
    torch.cuda.synchronize()
    P_o, ps_o, lse_o = oracle.fwd(synth.to_numpy_bits(s), B, H, S, N, sink=sink.numpy(),
                                  want_lse=True)
    got = lse.cpu().numpy()
    assert np.all(got > np.log(N) - 0.02) and np.all(got < np.log(N + 1) + 0.02), got
    assert_lse_close(got, lse_o, f"lse N={N}")
    assert_close(synth.to_numpy_bits(P), P_o, f"P N={N}")
    assert_close(ps.cpu().numpy(), ps_o, "p_sink")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_long_rows_with_exclusion(dt):
    N = 70000
    log(f"long rows with exclusion: {dt} N={N}")
    long_case(dt, N, B=2, H=2, S=3, causal=True, kl=[40001, N], with_sink=True, seed=77)
    # a key length that cuts inside the first segment: the later segments
    # are neither read nor computed, and their P is written as +0
    long_case(dt, N, B=1, H=1, S=5, causal=True, kl=[12345], seed=79)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_long_row_geometries_identical(dt):
    # both segment sizes and a capped grid (workgroups looping over rows)
    N = 50001
    B, H, S = 1, 3, 4
    log(f"long-row geometries: {dt} N={N}")
    s = synth.normal((B, H, S, N), 2.0, 500, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 501, "cpu", dt).to(dev())
    sink = synth.normal((H,), 1.0, 502, "cpu").to(dev())
    ref = run(s, g, sink=sink, causal=True)
    for cpl in STREAM_CPLS[dt]:
        for cap in (0, 5):
            assert run(s, g, launch=(4, cpl, 0, cap, 1), sink=sink, causal=True) == ref, (cpl, cap)
    if dt != torch.float32:
        for cap in (0, 5):
            assert run(s, g, launch=(8, 8, 0, cap, 1), sink=sink, causal=True) == ref, cap


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("N", [16385, 40000, 65536, 65544, 131072])
def test_wide_and_narrow_streaming_identical(dt, N):
    # rows of whole 16-byte chunks: the 8-wave workgroup (segments of 32,768
    # keys; the backward's default up to 65,536 keys) and the 4-wave one
    # (segments of 16,384 keys) give the same bytes, with mask, sink, causal
    # cut and lse, whatever each holds in registers, keeps in its LDS stash
    # or reads twice
    B, H, S = 1, 2, 3
    log(f"wide vs narrow streaming: {dt} N={N}")
    s = synth.normal((B, H, S, N), 2.0, 520, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 521, "cpu", dt).to(dev())
    mask = torch.zeros((B, 1, 1, N), device=dev())
    mask[..., N // 3:N // 3 + 777] = float("-inf")
    sink = synth.normal((H,), 1.0, 522, "cpu").to(dev())
    kw = dict(mask=mask, sink=sink, causal=True)
    ref = run(s, g, launch=(4, 8, 1, 0, 1), **kw)
    assert run(s, g, launch=(8, 8, 1, 0, 1), **kw) == ref
    assert run(s, g, **kw) == ref


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_key_lengths_at_segment_edges(dt):
    # Key lengths just below, at and just past the segment boundaries of
    # every streaming geometry (16-bit: 8,192 and 16,384 keys a segment with
    # 4 waves, 32,768 with 8; fp32: 8,192 and 16,384), so that the
    # last segment read is each of the ones the forward holds in registers,
    # keeps in its LDS stash or reads twice.  The bytes agree across
    # geometries, and with the oracle.
    N = 70000
    kl = [1, 8191, 8192, 16384, 16385, 32767, 32769, 49152, 49153, 65536, 65537, N]
    B, H, S = len(kl), 1, 2
    log(f"key lengths at segment edges: {dt} N={N}")
    s = synth.normal((B, H, S, N), 2.0, 530, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 531, "cpu", dt).to(dev())
    sink = synth.normal((H,), 1.0, 532, "cpu").to(dev())
    key_len = torch.tensor(kl, dtype=torch.int32, device=dev())
    ref = run(s, g, sink=sink, key_len=key_len)
    for cpl in STREAM_CPLS[dt]:
        assert run(s, g, launch=(4, cpl, 1, 0, 1), sink=sink, key_len=key_len) == ref, cpl
    if dt != torch.float32:
        assert run(s, g, launch=(8, 8, 1, 0, 1), sink=sink, key_len=key_len) == ref
    long_case(dt, N, B=B, H=H, S=S, with_sink=True, kl=kl, seed=533)


def test_long_rows_full_size_sampled():
    # long-context rows: bf16 [1,16,512,65536] (512 queries against 64K keys,
    # 2^29 elements) with the causal condition (key <= N - Sq + q) as a flag;
    # sampled rows against the oracle, stage-isolated backward on synthetic P
    B, H, S, N = 1, 16, 512, 65536
    log(f"bf16 [{B},{H},{S},{N}] causal flag, sampled rows")
    s = synth.normal((B, H, S, N), 2.0, 600, dev(), torch.bfloat16)
    P, _, lse = jas.fwd(s, causal=True, want_lse=True)
    torch.cuda.synchronize()
    idx = sample_rows(B * H * S, 24, seed=601)
    q = idx % S
    kend = q + (N - S) + 1
    k = len(idx)
    P_o, _, lse_o = oracle.fwd(gather_rows(s, idx).reshape(k, 1, 1, N), k, 1, 1, N,
                               key_len=kend.astype(np.int32), want_lse=True)
    assert_close(gather_rows(P, idx), P_o.reshape(k, N), "long P")
    assert_lse_close(lse.cpu().numpy()[idx], lse_o, "long lse")
    del P, s
    torch.cuda.empty_cache()
    Pin, gin, _ = synth.synthetic_bwd_inputs((B, H, S, N), torch.bfloat16, 602, dev())
    dS, _ = jas.bwd(Pin, gin, causal=True)
    torch.cuda.synchronize()
    P_rows = gather_rows(Pin, idx)
    P_rows[np.arange(N)[None, :] >= kend[:, None]] = 0
    dS_o, _ = oracle_rows_bwd(P_rows, gather_rows(gin, idx), N)
    assert_bitexact(gather_rows(dS, idx), dS_o, "long dS")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_streaming_in_place_and_padded_rows(dt):
    # in place: pass 2 reads every segment again before it writes it (the
    # last segment first), so probs == scores and dscores == probs are safe;
    # padded rows (ld > N) keep the padding untouched; both give the bytes
    # of the plain call
    B, H, S, N = 1, 2, 3, 40000
    log(f"streaming in place and padded rows: {dt} N={N}")
    s = synth.normal((B, H, S, N), 2.0, 700, "cpu", dt).to(dev())
    g = synth.normal((B, H, S, N), 1.0, 701, "cpu", dt).to(dev())
    sink = synth.normal((H,), 1.0, 702, "cpu").to(dev())
    P0, ps0 = jas.fwd(s, sink=sink, causal=True)
    dS0, d0 = jas.bwd(P0, g, p_sink=ps0, causal=True)
    x = s.clone()
    jas.fwd(x, sink=sink, causal=True, out=x, p_sink=torch.empty_like(ps0))
    y = P0.clone()
    jas.bwd(y, g, p_sink=ps0, causal=True, out=y)
    torch.cuda.synchronize()
    assert synth.to_numpy_bits(x).tobytes() == synth.to_numpy_bits(P0).tobytes()
    assert synth.to_numpy_bits(y).tobytes() == synth.to_numpy_bits(dS0).tobytes()
    for pad in (8, 3):   # 16-byte rows stay on the vector path; 3 takes the element path
        ld = N + pad
        big = torch.full((B * H * S * ld,), 5.0, dtype=dt, device=dev())
        sv = big.view(B, H, S, ld)[..., :N]
        sv.copy_(s)
        pbig = torch.full_like(big, 7.0)
        pv = pbig.view(B, H, S, ld)[..., :N]
        jas.fwd(sv, sink=sink, causal=True, out=pv, p_sink=torch.empty_like(ps0))
        gbig = torch.full_like(big, 3.0)
        gv = gbig.view(B, H, S, ld)[..., :N]
        gv.copy_(g)
        dbig = torch.full_like(big, 9.0)
        dv = dbig.view(B, H, S, ld)[..., :N]
        jas.bwd(pv, gv, p_sink=ps0, causal=True, out=dv)
        torch.cuda.synchronize()
        assert synth.to_numpy_bits(pv.contiguous()).tobytes() == synth.to_numpy_bits(P0).tobytes()
        assert synth.to_numpy_bits(dv.contiguous()).tobytes() == synth.to_numpy_bits(dS0).tobytes()
        assert torch.all(pbig.view(B, H, S, ld)[..., N:] == 7.0)
        assert torch.all(dbig.view(B, H, S, ld)[..., N:] == 9.0)
