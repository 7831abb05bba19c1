"""GPU: the forward that keeps each wave's share of the mask row in registers
from one of its rows to the next (jas_launch_t.mask_in_registers).

RL-Kernel PR #453, Summary: a row's result must not depend on the launch
geometry.  Keeping the mask in registers changes only which workgroup reads
which rows and how often the mask is loaded, never the arithmetic, so every
output (P, p_sink, lse) must be byte-identical to the forward without it,
whatever the grid, the workgroup shape, the mask strides (a mask row shared
by a batch entry, or one per query, which reloads on every row), the visible
lengths (key lengths and the causal cut reload when they change) and the
dtype.  The default path of the headline shape takes this forward, so the
full-tensor parity tests of that shape check it against the oracle as well.
"""
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import synth
from tests.gpu_util import dev, log

pytestmark = pytest.mark.gpu


def outputs(s, launch, **kw):
    P, ps, lse = jas.fwd(s, launch=launch, want_lse=True, **kw)
    torch.cuda.synchronize()
    out = [synth.to_numpy_bits(P).tobytes(), lse.cpu().numpy().tobytes()]
    if ps is not None:
        out.append(ps.cpu().numpy().tobytes())
    return out


OFF = (2, 5, 2, 0, 0, 2)
ON = [(0, 0, 0, 0, 0, 1), (2, 5, 1, 7, 0, 1), (2, 5, 2, 3, 0, 1), (2, 5, 1, 1, 0, 1),
      (2, 5, 2, 0, 0, 1), (2, 3, 1, 5, 0, 1)]


def case(dt, B, H, S, N, mask_per_query=False, causal=False, key_len=None, sink=True, seed=0):
    s = synth.normal((B, H, S, N), 2.0, seed, "cpu", dt).to(dev())
    if mask_per_query:
        mask = synth.normal((B, 1, S, N), 1.0, seed + 1, "cpu").to(dev())
        mask[..., :, N - 37:] = float("-inf")
        strides = (S * N, 0, N)
    else:
        mask = synth.normal((B, 1, 1, N), 1.0, seed + 1, "cpu").to(dev())
        for b in range(B):
            mask[b, ..., N - 5 - 31 * b:] = float("-inf")
        strides = (N, 0, 0)
    kw = dict(mask=mask, mask_strides=strides, causal=causal,
              sink=synth.normal((H,), 1.0, seed + 2, "cpu").to(dev()) if sink else None,
              key_len=None if key_len is None else torch.tensor(key_len, dtype=torch.int32,
                                                                  device=dev()))
    ref = outputs(s, OFF, **kw)
    for geo in ON:
        if geo[1] and geo[0] * geo[1] < -(-N // 512):
            continue  # the waves' chunks do not hold the row
        assert outputs(s, geo, **kw) == ref, geo
    assert outputs(s, None, **kw) == ref  # the default, with or without it


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_shared_mask_rows(dt):
    # workgroups whose rows cross batch entries (each with its own mask row) and heads
    log(f"mask in registers, mask per batch entry: {dt}")
    case(dt, B=3, H=2, S=37, N=4352, seed=600)
    case(dt, B=2, H=3, S=11, N=2560, seed=610)


def test_mask_per_query_and_exclusion():
    log("mask in registers: per-query mask, key lengths, causal cut")
    case(torch.bfloat16, B=2, H=2, S=19, N=4352, mask_per_query=True, seed=620)
    case(torch.bfloat16, B=3, H=2, S=17, N=4352, key_len=[4352, 3001, 1], seed=630)
    case(torch.bfloat16, B=2, H=1, S=23, N=3072, causal=True, key_len=[3072, 2047], seed=640)


def test_default_on_headline_sized_call():
    # 16,384 rows or more with a mask shared by the queries: the default
    # takes the mask in registers; the bytes equal the forward without it
    B, H, S, N = 2, 4, 2048, 4352
    log(f"mask in registers by default: bf16 [{B},{H},{S},{N}]")
    d = jas.make_desc((B, H, S, N), jas.JAS_DTYPE_BF16, jas.JAS_FLAG_MASK, None, (N, 0, 0))
    st, p = jas.jas_launch_plan(d, 0)
    assert st == 0 and p.mask_in_registers == 1
    s = synth.normal((B, H, S, N), 2.0, 650, "cpu", torch.bfloat16).to(dev())
    mask = torch.zeros((B, 1, 1, N), device=dev())
    mask[1, ..., N - 200:] = float("-inf")
    kw = dict(mask=mask, mask_strides=(N, 0, 0))
    assert outputs(s, None, **kw) == outputs(s, OFF, **kw)


def test_unaligned_rows_fall_back():
    # rows that cannot take 16-byte accesses run the element-wise forward
    # with the same grid: same bytes
    B, H, S, N = 2, 2, 9, 4352
    log("mask in registers asked for on element-wise rows")
    base = synth.normal((B * H * S * N + 1,), 2.0, 660, "cpu", torch.bfloat16).to(dev())
    s = base[1:].view(B, H, S, N)  # 2-byte offset: not 16-byte aligned
    mask = synth.normal((B, 1, 1, N), 1.0, 661, "cpu").to(dev())
    kw = dict(mask=mask, mask_strides=(N, 0, 0))
    assert outputs(s, (2, 5, 1, 4, 0, 1), **kw) == outputs(s, OFF, **kw)
