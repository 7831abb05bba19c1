"""GPU: jas_bwd_noalloc, the backward for callers that cannot allocate
(code under HIP graph capture, tight serving loops, harnesses that forbid
allocation), called through the C ABI and checked against jas_bwd, the entry
point it varies, on the same inputs: dS and d_sink byte-identical.  Calls
come in a row, each later one smaller than the one before, so a stale share
left in the library's scratch by an earlier call would show; one call fills
the scratch to its limit, JAS_NOALLOC_MAX_ROWS rows."""
import numpy as np
import pytest
import torch

import deterministic_attention_softmax_amd as jas
import synth
from tests.gpu_util import dev, log

pytestmark = pytest.mark.gpu


def inputs(shape, dt, seed):
    P, g, ps = synth.synthetic_bwd_inputs(shape, dt, seed, dev(), with_sink=True)
    return P, g, ps


def both(shape, dt, seed, causal=False):
    """(jas_bwd's dS, d_sink), (jas_bwd_noalloc's dS, d_sink) on one input."""
    B, H, S, N = shape
    P, g, ps = inputs(shape, dt, seed)
    flags = jas.JAS_FLAG_SINK | (jas.JAS_FLAG_CAUSAL if causal else 0)
    code = {torch.bfloat16: jas.JAS_DTYPE_BF16, torch.float32: jas.JAS_DTYPE_F32,
            torch.float16: jas.JAS_DTYPE_F16}[dt]
    d = jas.make_desc(shape, code, flags)
    stream = torch.cuda.current_stream().cuda_stream
    # the entry point it varies, with a workspace of its own
    ws = torch.empty(jas.jas_bwd_workspace_bytes(d), dtype=torch.uint8, device=dev())
    dS_a = torch.empty_like(P)
    dsk_a = torch.empty(H, dtype=torch.float32, device=dev())
    st = jas.jas_bwd(d, P.data_ptr(), g.data_ptr(), None, ps.data_ptr(), dS_a.data_ptr(),
                     dsk_a.data_ptr(), ws.data_ptr(), ws.numel(), stream)
    assert st == 0, jas.STATUS.get(st, st)
    # the allocation-free entry point: no workspace argument
    dS_b = torch.full_like(P, float("nan"))
    dsk_b = torch.full((H,), float("nan"), dtype=torch.float32, device=dev())
    st = jas.jas_bwd_noalloc(d, P.data_ptr(), g.data_ptr(), None, ps.data_ptr(), dS_b.data_ptr(),
                             dsk_b.data_ptr(), stream)
    assert st == 0, jas.STATUS.get(st, st)
    torch.cuda.synchronize()
    return (dS_a, dsk_a), (dS_b, dsk_b)


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_noalloc_matches_bwd_on_calls_in_a_row():
    cases = [
        ((1, 16, 65536, 64), torch.bfloat16, 900, False),   # JAS_NOALLOC_MAX_ROWS rows exactly
        ((2, 3, 500, 4352), torch.bfloat16, 901, False),
        ((2, 3, 97, 1000), torch.float32, 902, True),
        ((1, 2, 33, 700), torch.float16, 903, False),        # smaller again
    ]
    assert 16 * 65536 == jas.JAS_NOALLOC_MAX_ROWS
    for shape, dt, seed, causal in cases:
        log(f"jas_bwd_noalloc vs jas_bwd: {dt} {shape} causal={causal}")
        (dS_a, dsk_a), (dS_b, dsk_b) = both(shape, dt, seed, causal)
        assert same(dS_a, dS_b), f"dS differs {shape}"
        assert same(dsk_a, dsk_b), f"d_sink differs {shape}: {dsk_a} {dsk_b}"
        assert torch.isfinite(dsk_b).all()


def test_noalloc_without_sink_and_over_the_limit():
    # without a sink nothing goes to the scratch; over the limit with a sink
    # the call is refused and nothing is written
    shape = (1, 2, 40, 512)
    P, g, _ = inputs(shape, torch.bfloat16, 910)
    d = jas.make_desc(shape, jas.JAS_DTYPE_BF16, 0)
    stream = torch.cuda.current_stream().cuda_stream
    dS = torch.empty_like(P)
    assert jas.jas_bwd_noalloc(d, P.data_ptr(), g.data_ptr(), None, None, dS.data_ptr(), None,
                               stream) == 0
    ref, _ = jas.bwd(P, g)
    torch.cuda.synchronize()
    assert same(dS, ref)
    S = jas.JAS_NOALLOC_MAX_ROWS + 1
    big = jas.make_desc((1, 1, S, 8), jas.JAS_DTYPE_BF16, jas.JAS_FLAG_SINK)
    x = torch.zeros((1, 1, S, 8), dtype=torch.bfloat16, device=dev())
    ps = torch.zeros(S, dtype=torch.float32, device=dev())
    dsk = torch.full((1,), 7.0, dtype=torch.float32, device=dev())
    out = torch.full_like(x, 3.0)
    assert jas.jas_bwd_noalloc(big, x.data_ptr(), x.data_ptr(), None, ps.data_ptr(),
                               out.data_ptr(), dsk.data_ptr(), stream) == 10
    torch.cuda.synchronize()
    assert float(dsk[0]) == 7.0 and bool((out == 3.0).all())
