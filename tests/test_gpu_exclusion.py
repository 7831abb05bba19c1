"""GPU: causal and key-length exclusion (keys past a row's visible prefix are
neither read nor computed on).

RL-Kernel PR #240 (Prefill / Decode): a query sees key j when
j <= N - Sq + q; the same page's Path Status: text padding is cut per batch
entry, a row left with no key is all +0.  With JAS_FLAG_CAUSAL /
JAS_FLAG_KEY_LEN the library reads no score (forward) and no probability
(backward) past the prefix, so those regions are filled with NaN here: the
forward must equal, byte for byte, the dense forward on -inf scores, the
backward the dense backward on +0 probabilities, and both the oracle's
exclusion (which reads nothing there either) to the usual bar.
"""
import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import oracle
import synth
from tests.gpu_util import (assert_bitexact, assert_close, assert_lse_close, dev, gather_rows,
                            log, oracle_rows_bwd, oracle_rows_fwd, sample_rows)
from tests.test_gpu_invariance import valid_geometries

pytestmark = pytest.mark.gpu


def visible(B, Sq, N, causal, key_len):
    """bool [B, 1, Sq, N]: the keys a row sees (the causal condition and the
    batch entry's key length)."""
    q = torch.arange(Sq).view(1, 1, Sq, 1)
    k = torch.arange(N).view(1, 1, 1, N)
    vis = torch.ones((B, 1, Sq, N), dtype=torch.bool)
    if causal:
        vis = vis & (k <= (N - Sq) + q)
    if key_len is not None:
        vis = vis & (k < torch.as_tensor(key_len, dtype=torch.int64).view(B, 1, 1, 1))
    return vis


def fill_hidden(t, vis, value):
    """A copy of t with `value` on the keys that `vis` hides."""
    return t.masked_fill(~vis.to(t.device), value)


def run_case(dt, B, H, Sq, N, causal, key_len, mask=None, mask_strides=None, sink=None,
             seed=0, launch=None, check_oracle=True):
    s = synth.normal((B, H, Sq, N), 2.0, seed, "cpu", dt)
    g = synth.normal((B, H, Sq, N), 1.0, seed + 1, "cpu", dt)
    vis = visible(B, Sq, N, causal, key_len)
    kl = None if key_len is None else torch.tensor(key_len, dtype=torch.int32, device=dev())
    md = None if mask is None else mask.to(dev())
    sd = None if sink is None else sink.to(dev())
    s_nan = fill_hidden(s, vis, float("nan")).to(dev())
    s_inf = fill_hidden(s, vis, float("-inf")).to(dev())
    # forward: exclusion on NaN-filled scores == dense on -inf scores
    P1, ps1, l1 = jas.fwd(s_nan, mask=md, mask_strides=mask_strides, sink=sd, causal=causal,
                          key_len=kl, launch=launch, want_lse=True)
    P2, ps2, l2 = jas.fwd(s_inf, mask=md, mask_strides=mask_strides, sink=sd, launch=launch,
                          want_lse=True)
    torch.cuda.synchronize()
    assert synth.to_numpy_bits(P1).tobytes() == synth.to_numpy_bits(P2).tobytes(), "P vs dense"
    assert l1.cpu().numpy().tobytes() == l2.cpu().numpy().tobytes(), "lse vs dense"
    if sink is not None:
        assert ps1.cpu().numpy().tobytes() == ps2.cpu().numpy().tobytes(), "p_sink vs dense"
    # backward: exclusion on NaN-filled P == dense on P (+0 there)
    P_nan = fill_hidden(P1, vis, float("nan"))
    dS1, d1 = jas.bwd(P_nan, g.to(dev()), p_sink=ps1, causal=causal, key_len=kl, launch=launch)
    dS2, d2 = jas.bwd(P1, g.to(dev()), p_sink=ps1, launch=launch)
    torch.cuda.synchronize()
    assert synth.to_numpy_bits(dS1).tobytes() == synth.to_numpy_bits(dS2).tobytes(), "dS vs dense"
    if sink is not None:
        assert d1.cpu().numpy().tobytes() == d2.cpu().numpy().tobytes(), "d_sink vs dense"
    if not check_oracle:
        return synth.to_numpy_bits(P1), synth.to_numpy_bits(dS1), l1.cpu().numpy()
    # the oracle's exclusion on the NaN-filled inputs
    kl_np = None if key_len is None else np.asarray(key_len, np.int32)
    m_np = None if mask is None else mask.cpu().numpy()
    k_np = None if sink is None else sink.cpu().numpy()
    P_o, ps_o, lse_o = oracle.fwd(synth.to_numpy_bits(s_nan), B, H, Sq, N, mask=m_np,
                                  mask_strides=mask_strides or (0, 0, 0), sink=k_np,
                                  causal=causal, key_len=kl_np, want_lse=True)
    assert_close(synth.to_numpy_bits(P1), P_o, "P")
    assert_lse_close(l1.cpu().numpy(), lse_o)
    if sink is not None:
        assert_close(ps1.cpu().numpy(), ps_o, "p_sink")
    # stage-isolated backward: the oracle's P, NaN past the prefix, on both sides
    Pin = fill_hidden(synth.from_numpy_bits(P_o), vis, float("nan"))
    psin = None if sink is None else torch.from_numpy(ps_o).to(dev())
    dS, dsk = jas.bwd(Pin.to(dev()), g.to(dev()), p_sink=psin, causal=causal, key_len=kl,
                      launch=launch)
    torch.cuda.synchronize()
    dS_o, v_o = oracle.bwd(synth.to_numpy_bits(Pin), synth.to_numpy_bits(g), B, H, Sq, N,
                           p_sink=ps_o, causal=causal, key_len=kl_np)
    assert_bitexact(synth.to_numpy_bits(dS), dS_o, "dS")
    if sink is not None:
        assert_bitexact(dsk.cpu().numpy(), oracle.dsink(v_o, B, H, Sq), "d_sink")
    return synth.to_numpy_bits(P1), synth.to_numpy_bits(dS1), l1.cpu().numpy()


@pytest.mark.parametrize("Sq,N", [(600, 600), (64, 1000), (700, 300), (33, 4352), (5, 16384),
                                  (257, 257), (8, 8)])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_causal(dt, Sq, N):
    log(f"causal: {dt} Sq={Sq} N={N}")
    sink = synth.normal((2,), 1.0, Sq + N, "cpu")
    run_case(dt, 1, 2, Sq, N, True, None, sink=sink, seed=Sq * 7 + N)


@pytest.mark.parametrize("N", [700, 4352, 8449])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_key_len(dt, N):
    # full, a cut inside a chunk, one key, none, beyond N (clamped), negative
    kl = [N, 513, 1, 0, N + 100, -3]
    log(f"key_len: {dt} N={N} key_len={kl}")
    sink = synth.normal((3,), 1.0, N, "cpu")
    run_case(dt, len(kl), 3, 5, N, False, kl, sink=sink, seed=N)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_causal_key_len_mask_sink_together(dt):
    B, H, Sq, N = 3, 2, 40, 1300
    kl = [1300, 777, 1290]
    mask = synth.normal((B, 1, Sq, N), 1.0, 91, "cpu")
    mask[1, ..., 100:164] = float("-inf")
    sink = synth.normal((H,), 1.0, 92, "cpu")
    log(f"causal+key_len+mask+sink: {dt} [{B},{H},{Sq},{N}]")
    run_case(dt, B, H, Sq, N, True, kl, mask=mask, mask_strides=(Sq * N, 0, N), sink=sink,
             seed=93)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float32, torch.float16])
def test_elementwise_path(dt):
    # N not a multiple of a 16-byte chunk: the element-wise path
    log(f"exclusion, element-wise path: {dt}")
    sink = synth.normal((2,), 1.0, 95, "cpu")
    run_case(dt, 2, 2, 30, 1001, True, [1001, 517], sink=sink, seed=96)


@pytest.mark.parametrize("dt,N", [(torch.bfloat16, 4352), (torch.float32, 2000),
                                  (torch.float16, 1000)])
def test_every_launch_geometry_with_exclusion(dt, N):
    B, H, Sq = 2, 1, 9
    kl = [N - 37, 300]
    sink = synth.normal((H,), 1.0, 97, "cpu")
    geos = valid_geometries(dt, N)
    log(f"exclusion geometries: {dt} N={N}: {len(geos)}")
    ref = None
    for L in geos:
        cur = run_case(dt, B, H, Sq, N, True, kl, sink=sink, seed=98, launch=L,
                       check_oracle=ref is None)
        cur = (cur[0].tobytes(), cur[1].tobytes(), cur[2].tobytes())
        if ref is None:
            ref = cur
        else:
            assert cur == ref, f"launch {L} changed the bytes"


def test_causal_flag_1x32x8192x8192_sampled():
    # the causal self-attention workload with the flag: nothing above the
    # diagonal is read.  Forward on the -inf scores, sampled rows against the
    # oracle (each row's visible prefix as a -inf mask); backward on synthetic
    # P with nonzero values above the diagonal, which the flag must ignore.
    log("bf16 [1,32,8192,8192] causal flag + sink, sampled rows")
    B, H, S = 1, 32, 8192
    N = S
    s, sink, g = synth.causal_sink_bf16(seed=5, device=dev(), B=B, H=H, S=S)
    del g
    P, ps = jas.fwd(s, sink=sink, causal=True)
    torch.cuda.synchronize()
    rows = B * H * S
    idx = sample_rows(rows, 64, seed=51)
    idx = np.unique(np.concatenate([idx, [0, 1, rows - 1, 8191, 8192, 300]]))
    q = idx % S
    kend = q + 1
    hide = np.arange(N)[None, :] >= kend[:, None]
    m_rows = np.where(hide, -np.inf, 0.0).astype(np.float32)
    h_of = (idx // S) % H
    P_o, ps_o = oracle_rows_fwd(gather_rows(s, idx), N, mask_rows=m_rows,
                                sigma_rows=np.ascontiguousarray(sink.cpu().numpy()[h_of]))
    assert_close(gather_rows(P, idx), P_o, "causal-flag P")
    assert_close(ps.cpu().numpy()[idx], ps_o, "causal-flag p_sink")
    del P, ps, s
    torch.cuda.empty_cache()
    Pin, gin, psin = synth.synthetic_bwd_inputs((B, H, S, N), torch.bfloat16, 56, dev(),
                                                with_sink=True)
    dS, dsk = jas.bwd(Pin, gin, p_sink=psin, causal=True)
    torch.cuda.synchronize()
    ps_np = psin.cpu().numpy()
    P_rows = gather_rows(Pin, idx)
    P_rows[hide] = 0
    dS_o, _ = oracle_rows_bwd(P_rows, gather_rows(gin, idx), N,
                              ps_rows=np.ascontiguousarray(ps_np[idx]))
    assert_bitexact(gather_rows(dS, idx), dS_o, "causal-flag dS")
    dsk_np = dsk.cpu().numpy()
    for h in (0, H - 1):
        _, v_h = oracle.bwd(synth.to_numpy_bits(Pin[0, h]).reshape(1, 1, S, N),
                            synth.to_numpy_bits(gin[0, h]).reshape(1, 1, S, N), 1, 1, S, N,
                            p_sink=np.ascontiguousarray(ps_np[h * S:(h + 1) * S]), causal=True)
        assert_bitexact(dsk_np[h:h + 1], oracle.dsink(v_h, 1, 1, S), f"causal-flag d_sink[{h}]")


def test_key_len_joint_2x24x4352x4352_sampled():
    # joint attention with the text padding given as key lengths (batch 2 so
    # the two entries differ); sampled rows.  The backward runs on seeded
    # synthetic P, nonzero on the padded keys, which the key lengths hide.
    log("bf16 [2,24,4352,4352] key lengths, sampled rows")
    B, H, S, N = 2, 24, 4352, 4352
    s, _, g, pads = synth.joint_attention_bf16(seed=35, device=dev(), B=B, H=H, S=S, N=N)
    del g
    kl = torch.tensor([N - p for p in pads], dtype=torch.int32, device=dev())
    P, _ = jas.fwd(s, key_len=kl)
    torch.cuda.synchronize()
    idx = sample_rows(B * H * S, 64, seed=36)
    kend = np.asarray([N - p for p in pads])[idx // (H * S)]
    hide = np.arange(N)[None, :] >= kend[:, None]
    m_rows = np.where(hide, -np.inf, 0.0).astype(np.float32)
    P_o, _ = oracle_rows_fwd(gather_rows(s, idx), N, mask_rows=m_rows)
    assert_close(gather_rows(P, idx), P_o, "key_len P")
    del P, s
    Pin, gin, _ = synth.synthetic_bwd_inputs((B, H, S, N), torch.bfloat16, 37, dev())
    dS, _ = jas.bwd(Pin, gin, key_len=kl)
    torch.cuda.synchronize()
    P_rows = gather_rows(Pin, idx)
    P_rows[hide] = 0
    dS_o, _ = oracle_rows_bwd(P_rows, gather_rows(gin, idx), N)
    assert_bitexact(gather_rows(dS, idx), dS_o, "key_len dS")
