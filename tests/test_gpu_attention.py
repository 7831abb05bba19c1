"""GPU: the fused attention forward (QK on MFMA, the row softmax, PV on MFMA)
against the oracle's fixed-order attention.

RL-Kernel PR #453, Summary: the softmax between the QK GEMM and the AV GEMM;
RL-Kernel PR #240, Fixed Reduction Contract (one writer per score and per
output element, fixed accumulation order) and Path Status (MHA / MQA / GQA,
causal and padding masks).

The matrix cores accumulate in their own fixed order, not the oracle's
ascending one, so:
  * scores are within the bound of two binary32 summation orders,
    (D + 2) * 2^-24 * scale * sum_d |q_d k_d|;
  * P (written on request) is, byte for byte, jas_fwd of the kernel's own
    scores rounded to the dtype -- the softmax inside the fused kernel is the
    library's; lse and p_sink likewise;
  * the output is P.V of the kernel's own P within the binary32 sum's
    bound and one rounding;
  * the output is within a bound built from its sources of the oracle's:
    both sides round each p_j to the dtype once (u = 2^-8 bf16, 2^-11 fp16;
    a score difference can move a p_j across a rounding boundary on one side
    only, so 2u), the score and mask-add differences, both binary32 sums,
    fp16 subnormals, and the output's own rounding.
Invariance: a query's bytes do not depend on the batch or on its block, nor
on the launch's 16-query blocks per wavefront (1 or 2).
"""
import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import oracle
import synth
from tests.gpu_util import F32_ATOL, F32_RTOL, assert_lse_close, dev, log

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def raw_bytes(t):
    """A device tensor's bytes (any dtype, numpy has no bf16)."""
    return t.contiguous().view(torch.uint8).cpu().numpy().tobytes()


def draw(seed, B, H, Hkv, Sq, N, D, dt, std=1.0):
    q = synth.normal((B, H, Sq, D), std, seed, "cpu", dt)
    k = synth.normal((B, Hkv, N, D), std, seed + 1, "cpu", dt)
    v = synth.normal((B, Hkv, N, D), 1.0, seed + 2, "cpu", dt)
    return q, k, v


def check(q, k, v, scale, mask=None, mask_strides=None, sink=None, causal=False, kl=None, qb=0):
    B, H, Sq, D = q.shape
    Hkv, N = k.shape[1], k.shape[2]
    dt = q.dtype
    klt = None if kl is None else torch.tensor(kl, dtype=torch.int32, device=dev())
    r = jas.attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), scale=scale,
                     mask=None if mask is None else mask.to(dev()), mask_strides=mask_strides,
                     sink=None if sink is None else sink.to(dev()), causal=causal, key_len=klt,
                     want_lse=True, want_probs=True, want_scores=True, query_blocks=qb)
    torch.cuda.synchronize()
    o = oracle.attn_fwd(synth.to_numpy_bits(q), synth.to_numpy_bits(k), synth.to_numpy_bits(v),
                        np.float32(scale), mask=None if mask is None else mask.numpy(),
                        mask_strides=mask_strides or (0, 0, 0), causal=causal,
                        key_len=None if kl is None else np.array(kl, np.int32),
                        sink=None if sink is None else sink.numpy(), want_probs=True,
                        want_scores=True)
    # scores: two summation orders of the same exact products
    g = H // Hkv
    qf, kf, vf = f64(synth.to_numpy_bits(q)), f64(synth.to_numpy_bits(k)), f64(synth.to_numpy_bits(v))
    absS = np.zeros((B, H, Sq, N))
    for b in range(B):
        for h in range(H):
            absS[b, h] = abs(scale) * (np.abs(qf[b, h]) @ np.abs(kf[b, h // g]).T)
    S = r["scores"].cpu().numpy()
    err = np.abs(S.astype(np.float64) - o["scores"].astype(np.float64))
    assert np.all(err <= (D + 2) * U * absS + 1e-30), f"scores: worst {np.max(err / (absS + 1e-30))}"
    # the softmax inside the kernel is jas_fwd's, on the kernel's own scores
    Pf, psf, lsef = jas.fwd(r["scores"], mask=None if mask is None else mask.to(dev()),
                            mask_strides=mask_strides, sink=None if sink is None else sink.to(dev()),
                            causal=causal, key_len=klt, want_lse=True)
    torch.cuda.synchronize()
    want_P = synth.to_numpy_bits(Pf.to(dt))
    assert synth.to_numpy_bits(r["probs"]).tobytes() == want_P.tobytes(), "P is not jas_fwd(S)"
    assert r["lse"].cpu().numpy().tobytes() == lsef.cpu().numpy().tobytes()
    if sink is not None:
        assert r["p_sink"].cpu().numpy().tobytes() == psf.cpu().numpy().tobytes()
    assert_lse_close(r["lse"].cpu().numpy(), o["lse"], "lse vs oracle")
    # the output: the P.V of the kernel's own P, and the oracle's output
    u = 2.0 ** -8 if dt == torch.bfloat16 else 2.0 ** -11      # unit roundoff of the dtype
    # absolute error per rounded p_j: half the dtype's least subnormal (fp16),
    # or the binary32 softmax's absolute floor near its flush point (bf16)
    eta = F32_ATOL if dt == torch.bfloat16 else 2.0 ** -25
    Pg, Po = f64(synth.to_numpy_bits(r["probs"])), f64(o["probs"])
    mass_g, mass_o, exact_g = (np.zeros((B, H, Sq, D)) for _ in range(3))
    sum_v = np.zeros((B, H, 1, D))
    for b in range(B):
        for h in range(H):
            va = np.abs(vf[b, h // g])
            mass_g[b, h], mass_o[b, h] = Pg[b, h] @ va, Po[b, h] @ va
            exact_g[b, h] = Pg[b, h] @ vf[b, h // g]
            sum_v[b, h, 0] = va.sum(axis=0)
    got = f64(synth.to_numpy_bits(r["out"]))
    want = f64(o["out"])
    # binary32 sums of exact products: n additions in sequence err by at most
    # gamma_n = n*U/(1 - n*U) of the sum of magnitudes; the matrix cores add
    # 32-key steps to one accumulator (n <= N/32 + 32), the oracle key by key
    n_g = -(-N // 32) + 32
    gam_g, gam_o = n_g * U / (1 - n_g * U), N * U / (1 - N * U)
    lim_g = u * np.abs(got) * (1 + 2 * u) + gam_g * mass_g + 2 * eta
    bad = np.count_nonzero(~(np.abs(got - exact_g) <= lim_g))
    assert bad == 0, f"out is not P.V of the kernel's P: {bad} elements"
    # against the oracle.  Each side rounds its binary32 p_j to the dtype once
    # (|fl(p) - p| <= u*p + eta), so a score difference can move one p_j across
    # a rounding boundary on one side only: |P_g - P_o| <= 2u*p + 2*eta +
    # |p_g - p_o|.  The two binary32 p_j differ by the softmax's own agreement
    # with the oracle on equal inputs (F32_RTOL, the fp32 softmax bound)
    # and by exp(2*dx) - 1, dx the row's largest difference of s_j + mask_j
    # (the score bound above plus one rounding of the mask add on each side).
    mmax = 0.0 if mask is None else float(np.max(np.abs(np.nan_to_num(
        mask.numpy(), neginf=0.0)), initial=0.0))
    dx = (D + 4) * U * absS.max(axis=3, keepdims=True) + 2 * U * mmax
    rel_p = F32_RTOL + np.expm1(2 * dx)
    lim = (u * (np.abs(got) + np.abs(want)) * (1 + 2 * u)
           + (2 * u + rel_p + gam_g + gam_o) * (1 + 4 * u) * mass_o
           + 4 * eta * sum_v + 2 * eta)
    bad = np.count_nonzero(~(np.abs(got - want) <= lim))
    assert bad == 0, f"out: {bad} elements outside tolerance, worst {np.max(np.abs(got - want) / lim)}"
    return r


@pytest.mark.parametrize("qb", [1, 2])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("shape", [(1, 2, 2, 16, 256), (2, 4, 4, 37, 600), (1, 4, 1, 5, 1000),
                                   (1, 2, 2, 1, 1), (1, 6, 2, 33, 257), (1, 2, 1, 150, 300)])
def test_attention_against_oracle(shape, dt, D, qb):
    B, H, Hkv, Sq, N = shape
    log(f"attention {dt} B={B} H={H} Hkv={Hkv} Sq={Sq} N={N} D={D} query blocks {qb}")
    q, k, v = draw(Sq * 7 + N + D, B, H, Hkv, Sq, N, D, dt)
    check(q, k, v, 1.0 / np.sqrt(D), qb=qb)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_attention_mask_sink_causal_key_len(dt):
    B, H, Hkv, Sq, N, D = 2, 4, 2, 40, 700, 128
    q, k, v = draw(31, B, H, Hkv, Sq, N, D, dt, std=1.5)
    mask = torch.zeros((B, 1, 1, N))
    mask[0, ..., 650:] = float("-inf")
    mask[1, ..., :3] = -1.5
    sink = synth.normal((H,), 1.0, 32, "cpu")
    for qb in (1, 2):
        log(f"attention {dt} with mask, sink, causal, key lengths; query blocks {qb}")
        check(q, k, v, 0.09, mask=mask, mask_strides=(N, 0, 0), sink=sink, causal=True,
              kl=[700, 420], qb=qb)
        check(q, k, v, 0.09, sink=sink, kl=[0, 5], qb=qb)  # an empty batch entry: P = 0, p_sink = 1
        check(q, k, v, 0.09, causal=True, qb=qb)           # Sq < N: the last queries see all keys


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_attention_mask_rows_per_head_and_query(dt, D):
    # one mask row per (batch, head, query) at an odd row stride, so rows
    # start on 4-byte boundaries only (the kernel reads the mask 16 bytes at
    # a time), with -inf entries and a causal cut
    B, H, Hkv, Sq, N = 2, 3, 3, 37, 333
    ld = N + 1
    q, k, v = draw(71 + D, B, H, Hkv, Sq, N, D, dt, std=1.2)
    mask = synth.normal((B * H * Sq * ld,), 1.0, 72 + D, "cpu")
    mask[::7] = float("-inf")
    log(f"attention {dt} D={D}: mask rows per head and query, row stride {ld}")
    check(q, k, v, 0.1, mask=mask, mask_strides=(H * Sq * ld, Sq * ld, ld), causal=True)
    # the mask broadcast over queries, one row per head
    mh = synth.normal((H * N + 3,), 2.0, 73 + D, "cpu")
    check(q, k, v, 0.1, mask=mh, mask_strides=(0, N + 1, 0))


def test_attention_more_queries_than_keys_causal():
    # queries before the first visible key are fully masked rows: out = 0
    B, H, Sq, N, D = 1, 2, 50, 30, 64
    q, k, v = draw(41, B, H, H, Sq, N, D, torch.bfloat16)
    r = check(q, k, v, 0.125, causal=True)
    assert torch.all(r["out"][:, :, :Sq - N] == 0)


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_attention_at_the_key_limit(dt):
    # 16,384 keys, the most one call takes: 64 tiles of maxima per wave in
    # LDS; grouped heads, a mask, the sink and the causal cut, a ragged
    # query block
    B, H, Hkv, Sq, N, D = 1, 2, 1, 70, 16384, 128
    log(f"attention at the key limit: {dt} N={N}")
    q, k, v = draw(91, B, H, Hkv, Sq, N, D, dt)
    mask = synth.normal((B, 1, 1, N), 1.0, 92, "cpu")
    mask[..., 5000:5300] = float("-inf")
    sink = synth.normal((H,), 1.0, 93, "cpu")
    check(q, k, v, 1.0 / np.sqrt(D), mask=mask, mask_strides=(N, 0, 0), sink=sink, causal=True)


def test_attention_two_blocks_at_their_lds_limit():
    # 14,336 keys (56 tiles) at head dim 128: two query blocks' tile maxima
    # bring the workgroup's LDS to exactly 64 KB, the most the library gives
    # them; against the oracle, and the same bytes as one block
    B, H, Hkv, Sq, N, D = 1, 2, 1, 70, 14336, 128
    log(f"attention at the two-block LDS limit: N={N}")
    q, k, v = draw(95, B, H, Hkv, Sq, N, D, torch.bfloat16)
    mask = synth.normal((B, 1, 1, N), 1.0, 96, "cpu")
    mask[..., 9000:9100] = float("-inf")
    sink = synth.normal((H,), 1.0, 97, "cpu")
    check(q, k, v, 1.0 / np.sqrt(D), mask=mask, mask_strides=(N, 0, 0), sink=sink, causal=True,
          qb=2)
    rs = [jas.attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), mask=mask.to(dev()),
                       mask_strides=(N, 0, 0), sink=sink.to(dev()), causal=True, want_lse=True,
                       query_blocks=qb) for qb in (1, 2)]
    torch.cuda.synchronize()
    for key in ("out", "lse", "p_sink"):
        assert raw_bytes(rs[0][key]) == raw_bytes(rs[1][key]), key


def test_attention_batch_and_block_invariance():
    # a (batch, head)'s bytes do not move with the batch around it, nor with
    # the other query blocks of the call
    H, Hkv, Sq, N, D = 4, 2, 48, 900, 128
    q1, k1, v1 = draw(51, 1, H, Hkv, Sq, N, D, torch.bfloat16)
    r1 = jas.attn_fwd(q1.to(dev()), k1.to(dev()), v1.to(dev()), want_lse=True)
    qo, ko, vo = draw(52, 3, H, Hkv, Sq, N, D, torch.bfloat16)
    qo[1], ko[1], vo[1] = q1[0], k1[0], v1[0]
    r3 = jas.attn_fwd(qo.to(dev()), ko.to(dev()), vo.to(dev()), want_lse=True)
    r16 = jas.attn_fwd(q1[:, :, :16].contiguous().to(dev()), k1.to(dev()), v1.to(dev()))
    torch.cuda.synchronize()
    assert synth.to_numpy_bits(r3["out"][1]).tobytes() == synth.to_numpy_bits(r1["out"][0]).tobytes()
    assert r3["lse"].view(3, H, Sq)[1].cpu().numpy().tobytes() == r1["lse"].cpu().numpy().tobytes()
    assert synth.to_numpy_bits(r16["out"]).tobytes() == \
        synth.to_numpy_bits(r1["out"][:, :, :16].contiguous()).tobytes()


def test_joint_attention_1x24x4352x128_sampled():
    # the joint image+text attention shape (24 heads, 4,096 image + 256 text
    # keys, head dim 128) with the per-batch padding mask; 4 sampled queries
    # per head against the oracle
    B, H, S, D = 1, 24, 4352, 128
    log("fused attention bf16 [1,24,4352,128], padding mask, sampled queries")
    q = synth.normal((B, H, S, D), 1.0, 61, dev(), torch.bfloat16)
    k = synth.normal((B, H, S, D), 1.0, 62, dev(), torch.bfloat16)
    v = synth.normal((B, H, S, D), 1.0, 63, dev(), torch.bfloat16)
    mask = torch.zeros((B, 1, 1, S), device=dev())
    mask[..., S - 77:] = float("-inf")
    r = jas.attn_fwd(q, k, v, mask=mask, mask_strides=(S, 0, 0), want_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(64)
    qi = np.sort(rng.choice(S, 4, replace=False))
    qs = q[:, :, torch.as_tensor(qi, device=dev())].contiguous()
    o = oracle.attn_fwd(synth.to_numpy_bits(qs), synth.to_numpy_bits(k), synth.to_numpy_bits(v),
                        np.float32(1.0 / np.sqrt(D)), mask=mask.cpu().numpy(),
                        mask_strides=(S, 0, 0), want_probs=True)
    got = f64(synth.to_numpy_bits(r["out"][:, :, torch.as_tensor(qi, device=dev())]))
    want = f64(o["out"])
    Po = f64(o["probs"])
    vf = f64(synth.to_numpy_bits(v))
    mass = np.einsum("bhqk,bhkd->bhqd", Po, np.abs(vf))
    assert np.all(np.abs(got - want) <= 2.0 ** -8 * (mass + np.abs(want)) + 1e-30)
    lse = r["lse"].view(B, H, S)[:, :, torch.as_tensor(qi, device=dev())].cpu().numpy().reshape(-1)
    assert_lse_close(lse, o["lse"], "joint lse")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_attention_query_blocks_identical(dt, D):
    # the fast path (no P / score output) with 1 and 2 blocks of 16 queries
    # per wavefront and the library's own choice: identical bytes of out,
    # lse and p_sink, on ragged query counts, grouped heads, a mask shared by
    # the queries, the sink, the causal cut with Sq != N and key lengths
    B, H, Hkv, N = 2, 4, 2, 777
    for Sq, causal, kl, use_mask in ((1, False, None, False), (130, True, [777, 300], True),
                                     (200, False, [5, 777], True), (777, True, None, False),
                                     (900, True, None, True)):
        log(f"attention {dt} D={D} Sq={Sq} causal={causal} key_len={kl}: query blocks 0 / 1 / 2")
        q, k, v = draw(Sq + 17 * D, B, H, Hkv, Sq, N, D, dt, std=1.3)
        q, k, v = q.to(dev()), k.to(dev()), v.to(dev())
        mask = None
        if use_mask:
            mask = synth.normal((B, 1, 1, N), 1.0, Sq + 5, dev())
            mask[0, ..., 400:460] = float("-inf")
        sink = synth.normal((H,), 1.0, Sq + 6, dev())
        klt = None if kl is None else torch.tensor(kl, dtype=torch.int32, device=dev())
        rs = [jas.attn_fwd(q, k, v, scale=0.1, mask=mask,
                           mask_strides=None if mask is None else (N, 0, 0), sink=sink,
                           causal=causal, key_len=klt, want_lse=True, query_blocks=qb)
              for qb in (0, 1, 2)]
        torch.cuda.synchronize()
        for key in ("out", "lse", "p_sink"):
            ref = raw_bytes(rs[1][key])
            assert raw_bytes(rs[0][key]) == ref, f"{key}: default != 1 block"
            assert raw_bytes(rs[2][key]) == ref, f"{key}: 2 blocks != 1 block"


def test_attention_query_blocks_per_query_mask():
    # a mask that varies by query runs one block whatever is asked: the same
    # bytes for 0, 1 and 2, and P still jas_fwd of the scores (oracle check
    # with two blocks asked)
    B, H, Hkv, Sq, N, D = 1, 2, 2, 140, 500, 128
    q, k, v = draw(77, B, H, Hkv, Sq, N, D, torch.bfloat16)
    mask = synth.normal((B * H * Sq * N,), 1.0, 78, "cpu")
    mask[::5] = float("-inf")
    strides = (H * Sq * N, Sq * N, N)
    log("attention with a per-query mask: query blocks 0 / 1 / 2")
    rs = [jas.attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), scale=0.1, mask=mask.to(dev()),
                       mask_strides=strides, want_lse=True, query_blocks=qb) for qb in (0, 1, 2)]
    torch.cuda.synchronize()
    for key in ("out", "lse"):
        ref = raw_bytes(rs[1][key])
        assert raw_bytes(rs[0][key]) == ref and raw_bytes(rs[2][key]) == ref, key
    check(q, k, v, 0.1, mask=mask, mask_strides=strides, qb=2)


def test_joint_attention_query_blocks_identical():
    # the joint image+text shape, where the library picks 2 blocks per
    # wavefront: the same bytes as with 1
    B, H, S, D = 1, 24, 4352, 128
    log("fused attention bf16 [1,24,4352,128], padding mask: query blocks 0 / 1 / 2")
    q = synth.normal((B, H, S, D), 1.0, 81, dev(), torch.bfloat16)
    k = synth.normal((B, H, S, D), 1.0, 82, dev(), torch.bfloat16)
    v = synth.normal((B, H, S, D), 1.0, 83, dev(), torch.bfloat16)
    mask = torch.zeros((B, 1, 1, S), device=dev())
    mask[..., S - 100:] = float("-inf")
    rs = [jas.attn_fwd(q, k, v, mask=mask, mask_strides=(S, 0, 0), want_lse=True, query_blocks=qb)
          for qb in (0, 1, 2)]
    torch.cuda.synchronize()
    for key in ("out", "lse"):
        ref = raw_bytes(rs[1][key])
        assert raw_bytes(rs[0][key]) == ref
        assert raw_bytes(rs[2][key]) == ref


def test_attention_prepared_call_matches_wrapper():
    # attn_fwd_prepared (checks done once, then one C call per run) writes
    # the bytes attn_fwd writes; running it twice changes nothing
    B, H, Hkv, Sq, N, D = 2, 4, 2, 150, 900, 128
    log("attention prepared call")
    q, k, v = draw(111, B, H, Hkv, Sq, N, D, torch.bfloat16)
    q, k, v = q.to(dev()), k.to(dev()), v.to(dev())
    mask = synth.normal((B, 1, 1, N), 1.0, 112, dev())
    sink = synth.normal((H,), 1.0, 113, dev())
    kw = dict(scale=0.1, mask=mask, mask_strides=(N, 0, 0), sink=sink, causal=True, want_lse=True)
    ref = jas.attn_fwd(q, k, v, **kw)
    run, res = jas.attn_fwd_prepared(q, k, v, **kw)
    for _ in range(2):
        run()
        torch.cuda.synchronize()
        for key in ("out", "lse", "p_sink"):
            assert raw_bytes(res[key]) == raw_bytes(ref[key]), key
