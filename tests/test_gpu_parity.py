"""GPU parity: the HIP library through its C ABI against the CPU oracle on the
same seeded inputs (RL-Kernel PR #453: every GPU backend checked against the
CPU reference of the same tile order; here the oracle in oracle/).

Forward: P and p_sink within the tolerance (1 ulp for bf16 and fp16, 4e-6
relative fp32), the row log-sum-exp within 4e-6 * max(1, |lse|);
the exponential is the hardware one on the GPU.  Backward, stage-isolated:
both sides read the same P, dP, p_sink (never a GPU output), dS and d_sink are
bit-exact.  Composed fwd->bwd chains are checked separately with a
condition-scaled bound.
"""
import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import oracle
import synth
from tests.gpu_util import (assert_bitexact, assert_close, assert_lse_close, dev, gather_rows,
                            log, oracle_rows_bwd, oracle_rows_fwd, sample_rows)
from tests.ref64 import bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def run_fwd_bwd_full(s, g, mask=None, mask_strides=None, sink=None, launch=None):
    """GPU fwd on s; GPU bwd on the oracle's P (stage-isolated); compare all."""
    B, H, S, N = s.shape
    s_np = synth.to_numpy_bits(s)
    m_np = None if mask is None else mask.cpu().numpy()
    k_np = None if sink is None else sink.cpu().numpy()
    P, ps, lse = jas.fwd(s.to(dev()), mask=None if mask is None else mask.to(dev()),
                         mask_strides=mask_strides, sink=None if sink is None else sink.to(dev()),
                         launch=launch, want_lse=True)
    torch.cuda.synchronize()
    P_o, ps_o, lse_o = oracle.fwd(s_np, B, H, S, N, mask=m_np,
                                  mask_strides=mask_strides or (0, 0, 0), sink=k_np,
                                  want_lse=True)
    worst = assert_close(synth.to_numpy_bits(P), P_o, "P")
    if sink is not None:
        assert_close(ps.cpu().numpy(), ps_o, "p_sink")
    assert_lse_close(lse.cpu().numpy(), lse_o)
    # backward on the oracle's P
    g_np = synth.to_numpy_bits(g)
    Pin = synth.from_numpy_bits(P_o, dev())
    psin = None if sink is None else torch.from_numpy(ps_o).to(dev())
    dS, dsk = jas.bwd(Pin, g.to(dev()), p_sink=psin, launch=launch)
    torch.cuda.synchronize()
    dS_o, v_o = oracle.bwd(P_o, g_np, B, H, S, N, p_sink=ps_o)
    assert_bitexact(synth.to_numpy_bits(dS), dS_o, "dS")
    if sink is not None:
        assert_bitexact(dsk.cpu().numpy(), oracle.dsink(v_o, B, H, S), "d_sink")
    return worst


def test_grad_check_fp32_2x4x257x257():
    # fp32 scores [2,4,257,257] ~ N(0, 3^2), dP ~ N(0,1); two tiles, tail of 1
    log("fp32 [2,4,257,257] fwd+bwd")
    s, g = synth.grad_check_fp32(seed=1)
    run_fwd_bwd_full(s, g)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_16bit_2x4x257x257_with_mask_and_sink(dt):
    log(f"{dt} [2,4,257,257] with per-batch mask and sink")
    s, g = synth.grad_check_fp32(seed=11)
    s, g = s.to(dt), g.to(dt)
    mask = torch.zeros((2, 1, 1, 257))
    mask[0, ..., 200:] = float("-inf")
    mask[1, ..., 256:] = float("-inf")
    sink = synth.normal((4,), 1.0, 12, "cpu")
    run_fwd_bwd_full(s, g, mask=mask, mask_strides=(257, 0, 0), sink=sink)


@pytest.mark.parametrize("N", [1, 7, 8, 255, 256, 257, 511, 513, 1000, 4352, 8449, 16384])
@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16])
def test_row_lengths(N, dt):
    rows = 24 if N <= 4352 else 6
    log(f"row lengths: {dt} N={N} rows={rows}")
    s = synth.normal((1, 2, rows // 2, N), 3.0, N, "cpu", dt)
    g = synth.normal((1, 2, rows // 2, N), 1.0, N + 1, "cpu", dt)
    sink = synth.normal((2,), 1.0, N + 2, "cpu")
    run_fwd_bwd_full(s, g, sink=sink)


@pytest.mark.parametrize("N", [4353, 4374, 4522, 4608, 8705, 9169, 9196, 9216])
def test_fp32_rows_at_the_chunk_size_limits(N):
    # fp32 rows of 18 and of 35 to 36 tiles: one or two wavefronts' largest
    # compiled register share (17 chunks per lane) no longer holds the row,
    # so the default geometry takes more wavefronts per row
    log(f"fp32 N={N} at the chunk-size limits")
    s = synth.normal((1, 2, 3, N), 3.0, N, "cpu", torch.float32)
    g = synth.normal((1, 2, 3, N), 1.0, N + 1, "cpu", torch.float32)
    sink = synth.normal((2,), 1.0, N + 2, "cpu")
    run_fwd_bwd_full(s, g, sink=sink)


def test_rows_16384x4352_forward_all_rows():
    # bf16 [1,1,16384,4352], N(0,1) scaled by sqrt(128) then 1/sqrt(128), x8 on 0.1%
    log("bf16 16384 x 4352 forward, all rows")
    s = synth.rows_with_outliers_bf16(seed=2, device=dev())
    P, _ = jas.fwd(s)
    torch.cuda.synchronize()
    s_np = synth.to_numpy_bits(s)
    P_o, _ = oracle.fwd(s_np, 1, 1, 16384, 4352)
    worst = assert_close(synth.to_numpy_bits(P), P_o, "16384x4352 P")
    log(f"16384 x 4352: max {worst} bf16 ulp")


def compare_rows(got, want, what, bitexact=False, chunk=8192):
    """got / want: host bit arrays of the same [rows, N] layout, compared in
    row chunks (bounded host memory) at the parity bar."""
    got, want = got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1])
    assert got.shape == want.shape, what
    worst = 0
    for r0 in range(0, got.shape[0], chunk):
        sl = slice(r0, r0 + chunk)
        if bitexact:
            assert_bitexact(got[sl], want[sl], f"{what} rows {r0}..")
        else:
            worst = max(worst, assert_close(got[sl], want[sl], f"{what} rows {r0}.."))
    return worst


def test_joint_attention_1x24x4352x4352_all_rows():
    # the headline workload, whole: bf16 [1,24,4352,4352] ~ N(0, 2^2) with the
    # per-batch text padding mask and its dP, at the launch the benchmark
    # times (default geometry).  Every one of the 104,448 rows: P within 1
    # bf16 ulp of the oracle; then the backward, stage-isolated on the
    # oracle's P and the workload's dP, bit-exact on every row
    log("bf16 [1,24,4352,4352] mask fwd + bwd, all 104,448 rows")
    B, H, S, N = 1, 24, 4352, 4352
    s, mask, g, pads = synth.joint_attention_bf16(seed=3, device=dev(), B=B, H=H, S=S, N=N)
    P, _ = jas.fwd(s, mask=mask.view(B, 1, 1, N), mask_strides=(N, 0, 0))
    torch.cuda.synchronize()
    P_o, _ = oracle.fwd(synth.to_numpy_bits(s), B, H, S, N, mask=mask.cpu().numpy(),
                        mask_strides=(N, 0, 0))
    worst = compare_rows(synth.to_numpy_bits(P), P_o, "joint P")
    log(f"joint P: all rows within {worst} bf16 ulp")
    del P, s
    Pin = synth.from_numpy_bits(P_o, dev())
    dS, _ = jas.bwd(Pin, g)
    torch.cuda.synchronize()
    dS_o, _ = oracle.bwd(P_o, synth.to_numpy_bits(g), B, H, S, N)
    compare_rows(synth.to_numpy_bits(dS), dS_o, "joint dS", bitexact=True)


def test_joint_attention_batch2_all_rows():
    # the per-batch mask with B=2 (different padding per batch entry), smaller S
    log("bf16 [2,3,96,4352] per-batch mask fwd+bwd, all rows")
    s, mask, g, pads = synth.joint_attention_bf16(seed=34, device="cpu", B=2, H=3, S=96, N=4352)
    assert pads[0] != pads[1]
    run_fwd_bwd_full(s, g, mask=mask.view(2, 1, 1, 4352), mask_strides=(4352, 0, 0))


def test_causal_sink_1x32x8192x8192_four_full_heads():
    # bf16 causal [1,32,8192,8192] + per-head sink, 2^31 elements (64-bit
    # offsets), full-size launches.  Every row of four heads (first, last
    # and two between), taken head by head to bound host memory: P and
    # p_sink against the oracle; then the backward of the whole tensor on
    # those heads' oracle P and p_sink (the other heads get seeded synthetic
    # inputs), dS of every row of the four heads and their d_sink bit-exact
    log("bf16 [1,32,8192,8192] causal+sink fwd + bwd + d_sink, every row of 4 heads")
    B, H, S = 1, 32, 8192
    N = S
    heads = (0, 11, 22, H - 1)
    s, sink, g = synth.causal_sink_bf16(seed=5, device=dev(), B=B, H=H, S=S)
    P, ps = jas.fwd(s, sink=sink)
    torch.cuda.synchronize()
    sk = sink.cpu().numpy()
    Pin, _, psin = synth.synthetic_bwd_inputs((B, H, S, N), torch.bfloat16, 55, dev(),
                                              with_sink=True, zero_upper=True)
    for h in heads:
        P_o, ps_o = oracle.fwd(synth.to_numpy_bits(s[0, h]).reshape(1, 1, S, N), 1, 1, S, N,
                               sink=np.ascontiguousarray(sk[h:h + 1]))
        worst = compare_rows(synth.to_numpy_bits(P[0, h]), P_o, f"causal P head {h}")
        assert_close(ps[h * S:(h + 1) * S].cpu().numpy(), ps_o, f"causal p_sink head {h}")
        log(f"causal head {h}: P within {worst} bf16 ulp")
        Pin[0, h] = synth.from_numpy_bits(P_o.reshape(S, N), dev())
        psin[h * S:(h + 1) * S] = torch.from_numpy(ps_o).to(dev())
    del P, ps, s
    torch.cuda.empty_cache()
    dS, dsk = jas.bwd(Pin, g, p_sink=psin)
    torch.cuda.synchronize()
    dsk_np = dsk.cpu().numpy()
    ps_np = psin.cpu().numpy()
    for h in heads:
        P_h = synth.to_numpy_bits(Pin[0, h]).reshape(1, 1, S, N)
        dS_o, v_h = oracle.bwd(P_h, synth.to_numpy_bits(g[0, h]).reshape(1, 1, S, N), 1, 1, S, N,
                               p_sink=np.ascontiguousarray(ps_np[h * S:(h + 1) * S]))
        compare_rows(synth.to_numpy_bits(dS[0, h]), dS_o, f"causal dS head {h}", bitexact=True)
        assert_bitexact(dsk_np[h:h + 1], oracle.dsink(v_h, 1, 1, S), f"causal d_sink[{h}]")


def test_composed_chain_condition_scaled():
    # GPU fwd -> GPU bwd against oracle fwd -> oracle bwd: P may differ by one
    # bf16 ulp, which cancellation in dP - delta can amplify, so the bound
    # scales with the conditioning: |d dS_j| <= tol*(|dS_j| + P_j(|dP_j| + |delta|))
    log("composed: bf16 [1,4,64,4352] fwd->bwd with sink")
    B, H, S, N = 1, 4, 64, 4352
    s = synth.normal((B, H, S, N), 2.0, 70, "cpu", torch.bfloat16)
    g = synth.normal((B, H, S, N), 1.0, 71, "cpu", torch.bfloat16)
    sink = synth.normal((H,), 1.0, 72, "cpu")
    P, ps = jas.fwd(s.to(dev()), sink=sink.to(dev()))
    dS, dsk = jas.bwd(P, g.to(dev()), p_sink=ps)
    torch.cuda.synchronize()
    P_o, ps_o = oracle.fwd(synth.to_numpy_bits(s), B, H, S, N, sink=sink.numpy())
    dS_o, v_o = oracle.bwd(P_o, synth.to_numpy_bits(g), B, H, S, N, p_sink=ps_o)
    d_o = oracle.dsink(v_o, B, H, S)
    Pf = bf16_bits_to_f32(P_o).astype(np.float64).reshape(-1, N)
    gf = bf16_bits_to_f32(synth.to_numpy_bits(g)).astype(np.float64).reshape(-1, N)
    delta = (Pf * gf).sum(axis=1, keepdims=True)
    tol = 2.0 ** -7
    got = bf16_bits_to_f32(synth.to_numpy_bits(dS)).astype(np.float64).reshape(-1, N)
    want = bf16_bits_to_f32(dS_o).astype(np.float64).reshape(-1, N)
    lim = tol * (np.abs(want) + Pf * (np.abs(gf) + np.abs(delta))) + 1e-30
    assert np.all(np.abs(got - want) <= lim)
    vscale = np.abs(ps_o.astype(np.float64) * delta[:, 0]).reshape(B, H, S).sum(axis=(0, 2))
    assert np.all(np.abs(dsk.cpu().numpy() - d_o) <= tol * vscale + 1e-30)


def test_fp16_joint_attention_1x24x4352x4352_sampled():
    # the joint attention workload in fp16: full-size launch, sampled rows,
    # P, the row log-sum-exp, and the stage-isolated backward
    log("fp16 [1,24,4352,4352] mask fwd + lse; bwd on synthetic P; sampled rows")
    B, H, S, N = 1, 24, 4352, 4352
    s, mask, _, _ = synth.joint_attention_bf16(seed=3, device=dev(), B=B, H=H, S=S, N=N)
    s = s.to(torch.float16)
    P, _, lse = jas.fwd(s, mask=mask.view(B, 1, 1, N), mask_strides=(N, 0, 0), want_lse=True)
    torch.cuda.synchronize()
    idx = sample_rows(B * H * S, 96, seed=31)
    m_np = mask.cpu().numpy()
    k = len(idx)
    P_o, _, lse_o = oracle.fwd(gather_rows(s, idx).reshape(1, k, 1, N), 1, k, 1, N,
                               mask=np.ascontiguousarray(m_np[idx // (H * S)]),
                               mask_strides=(0, N, 0), want_lse=True)
    assert_close(gather_rows(P, idx), P_o.reshape(k, N), "fp16 joint P")
    assert_lse_close(lse.cpu().numpy()[idx], lse_o, "fp16 joint lse")
    del P, s
    Pin, gin, _ = synth.synthetic_bwd_inputs((B, H, S, N), torch.float16, 34, dev())
    dS, _ = jas.bwd(Pin, gin)
    torch.cuda.synchronize()
    dS_o, _ = oracle_rows_bwd(gather_rows(Pin, idx), gather_rows(gin, idx), N)
    assert_bitexact(gather_rows(dS, idx), dS_o, "fp16 joint dS")


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32])
def test_prepared_calls_match_wrapper(dt):
    # fwd_prepared / bwd_prepared (the checks done once, then one C call per
    # run) write the bytes fwd / bwd write, with the mask, the sink, the lse
    # and the causal cut; running them twice changes nothing
    B, H, S, N = 2, 3, 40, 700
    log(f"prepared calls {dt}")
    s = synth.normal((B, H, S, N), 2.0, 501, dev(), dt)
    g = synth.normal((B, H, S, N), 1.0, 502, dev(), dt)
    mask = synth.normal((B, 1, 1, N), 1.0, 503, dev())
    mask[1, ..., 600:] = float("-inf")
    sink = synth.normal((H,), 1.0, 504, dev())
    P_w, ps_w, lse_w = jas.fwd(s, mask=mask, sink=sink, causal=True, want_lse=True)
    dS_w, dsk_w = jas.bwd(P_w, g, p_sink=ps_w, causal=True)
    run_f, (P, ps, lse) = jas.fwd_prepared(s, mask=mask, sink=sink, causal=True, want_lse=True)
    run_b, (dS, dsk) = jas.bwd_prepared(P, g, p_sink=ps, causal=True)
    for _ in range(2):
        run_f()
        run_b()
        torch.cuda.synchronize()
        for a, b in ((P, P_w), (ps, ps_w), (lse, lse_w), (dS, dS_w), (dsk, dsk_w)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
