"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function declared in include/jas.h, and rejects bad arguments with the
documented status before any HIP call (nothing here reaches a launch)."""
import ctypes
import os
import re

import pytest

import deterministic_attention_softmax_amd as jas

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, never dereferenced device addresses (validation fails before any use)
A = 0x10000000
B_ = 0x20000000
C = 0x30000000
D = 0x40000000
E = 0x50000000
W = 0x60000000


def declared_functions():
    src = open(os.path.join(ROOT, "include", "jas.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(jas_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert {"jas_fwd", "jas_bwd", "jas_fwd_ex", "jas_bwd_ex", "jas_bwd_workspace_bytes",
            "jas_status_str", "jas_contract"} <= set(names)
    L = ctypes.CDLL(jas.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_contract_and_status_strings():
    c = jas.jas_contract()
    assert "tile=256" in c and "gfx950" in c and "atomics=none" in c
    assert "attn=" in c and "two-pass" in c
    for code in range(11):
        assert jas.jas_status_str(code) and jas.jas_status_str(code) != "unknown status"
    assert jas.jas_status_str(99) == "unknown status"


def desc(B=1, H=2, S=3, N=300, dtype=jas.JAS_DTYPE_BF16, flags=0, ld=None, ms=(0, 0, 0)):
    return jas.make_desc((B, H, S, N), dtype, flags, ld, ms)


def fwd(d, scores=A, mask=None, sink=None, probs=B_, p_sink=None, launch=None, key_len=None,
        lse=None):
    return jas.jas_fwd_ex(d, scores, mask, key_len, sink, probs, p_sink, lse, launch, None)


def bwd(d, probs=A, dprobs=B_, p_sink=None, dscores=C, d_sink=None, ws=None, ws_bytes=0,
        key_len=None):
    return jas.jas_bwd(d, probs, dprobs, key_len, p_sink, dscores, d_sink, ws, ws_bytes, None)


def test_null_desc_and_pointers():
    L = jas.lib()
    assert L.jas_fwd(None, A, None, None, None, B_, None, None, None) == 1
    assert L.jas_bwd(None, A, B_, None, None, C, None, None, 0, None) == 1
    assert fwd(desc(), scores=None) == 1
    assert fwd(desc(), probs=None) == 1
    assert bwd(desc(), probs=None) == 1
    assert bwd(desc(), dprobs=None) == 1
    assert bwd(desc(), dscores=None) == 1


def test_flag_pointer_predicates():
    # flag set, pointer missing -> NULL_POINTER; pointer given, flag unset -> BAD_FLAGS
    assert fwd(desc(flags=jas.JAS_FLAG_MASK)) == 1
    assert fwd(desc(flags=jas.JAS_FLAG_SINK), sink=C) == 1            # p_sink missing
    assert fwd(desc(flags=jas.JAS_FLAG_SINK), p_sink=D) == 1          # sink missing
    assert fwd(desc(), mask=C) == 4
    assert fwd(desc(), sink=C) == 4
    assert fwd(desc(), p_sink=D) == 4
    assert fwd(desc(flags=1 << 5)) == 4
    assert bwd(desc(flags=jas.JAS_FLAG_SINK), p_sink=D) == 1          # d_sink missing
    assert bwd(desc(), p_sink=D) == 4
    assert bwd(desc(), d_sink=E) == 4
    # key lengths: pointer iff JAS_FLAG_KEY_LEN
    assert fwd(desc(flags=jas.JAS_FLAG_KEY_LEN)) == 1
    assert fwd(desc(), key_len=W) == 4
    assert bwd(desc(flags=jas.JAS_FLAG_KEY_LEN)) == 1
    assert bwd(desc(), key_len=W) == 4
    assert fwd(desc(flags=1 << 5)) == 4
    # row log-sum-exp: pointer iff JAS_FLAG_LSE
    assert fwd(desc(flags=jas.JAS_FLAG_LSE)) == 1
    assert fwd(desc(), lse=W) == 4


def test_shapes_and_dtype():
    assert fwd(desc(N=0)) == 2
    assert fwd(desc(B=-1)) == 2
    assert fwd(desc(ld=299)) == 2
    assert fwd(desc(ms=(-1, 0, 0), flags=jas.JAS_FLAG_MASK), mask=C) == 2
    assert fwd(desc(N=jas.JAS_MAX_KEYS + 1)) == 7
    assert fwd(desc(dtype=7)) == 3
    assert fwd(desc(dtype=3)) == 3
    assert fwd(desc(dtype=jas.JAS_DTYPE_F16), scores=A + 1) == 9  # fp16 is a known dtype
    # rows * ld overflowing int64
    assert fwd(desc(B=1 << 40, H=1 << 20, S=1 << 10, N=8)) == 2


def test_alignment():
    assert fwd(desc(), scores=A + 1) == 9
    assert fwd(desc(dtype=jas.JAS_DTYPE_F32), probs=B_ + 2) == 9
    assert fwd(desc(flags=jas.JAS_FLAG_MASK), mask=C + 2) == 9
    assert bwd(desc(), dscores=C + 1) == 9
    assert fwd(desc(flags=jas.JAS_FLAG_KEY_LEN), key_len=W + 2) == 9
    assert fwd(desc(flags=jas.JAS_FLAG_LSE), lse=W + 2) == 9


def test_aliasing():
    # Every call here must fail validation: a call that passed would launch a
    # kernel on these fake addresses.
    d = desc(B=1, H=1, S=4, N=300)               # 4 rows x 600 bytes
    assert fwd(d, scores=A, probs=A + 600) == 5  # partial overlap
    assert fwd(d, scores=A, probs=A - 600) == 5
    dm = desc(B=1, H=1, S=4, N=300, flags=jas.JAS_FLAG_MASK, ms=(0, 0, 300))
    assert fwd(dm, mask=B_ + 4) == 5             # mask inside probs
    ds = desc(B=1, H=1, S=4, N=300, flags=jas.JAS_FLAG_SINK)
    assert fwd(ds, sink=C, p_sink=B_ + 8) == 5   # p_sink inside probs
    assert bwd(d, probs=A, dprobs=B_, dscores=A + 2) == 5
    dsb = desc(B=1, H=1, S=4, N=300, flags=jas.JAS_FLAG_SINK)
    ws = jas.jas_bwd_workspace_bytes(dsb)
    assert bwd(dsb, p_sink=D, d_sink=E, ws=D, ws_bytes=ws) == 5
    dk = desc(B=1, H=1, S=4, N=300, flags=jas.JAS_FLAG_KEY_LEN)
    assert fwd(dk, key_len=B_ + 64) == 5         # key lengths inside probs
    assert bwd(dk, key_len=C + 4) == 5           # key lengths inside dscores
    dl = desc(B=1, H=1, S=4, N=300, flags=jas.JAS_FLAG_LSE)
    assert fwd(dl, lse=B_ + 16) == 5             # lse inside probs
    assert fwd(dl, lse=A + 16) == 5              # lse inside scores
    dls = desc(B=1, H=1, S=4, N=300, flags=jas.JAS_FLAG_LSE | jas.JAS_FLAG_SINK)
    assert fwd(dls, sink=C, p_sink=D, lse=D + 8) == 5   # lse overlapping p_sink


def test_workspace():
    d = desc(B=2, H=3, S=5, flags=jas.JAS_FLAG_SINK)
    need = jas.jas_bwd_workspace_bytes(d)
    assert need == 256 and need >= 2 * 3 * 5 * 4
    assert jas.jas_bwd_workspace_bytes(desc(B=2, H=3, S=5)) == 0
    d2 = desc(B=1, H=1, S=1000, flags=jas.JAS_FLAG_SINK)
    assert jas.jas_bwd_workspace_bytes(d2) == 4096
    assert bwd(d, p_sink=D, d_sink=E, ws=None, ws_bytes=need) == 6
    assert bwd(d, p_sink=D, d_sink=E, ws=W, ws_bytes=need - 4) == 6
    # the size depends on shape and flags only
    L = jas.lib()
    assert L.jas_bwd_workspace_bytes(None) == 0


def test_launch_override_validation():
    d = desc(B=1, H=1, S=4, N=4352)  # 17 tiles -> 9 bf16 slots
    bad = [(3, 0, 0, 0), (1, 4, 0, 0), (1, 5, 0, 0), (2, 9, 3, 0), (-1, 0, 0, 0),
           # streaming: 4 waves, one row per workgroup, a streaming segment size
           (0, 3, 0, 0, 1), (2, 0, 0, 0, 1), (0, 0, 2, 0, 1), (0, 0, 0, 0, 2), (0, 9, 0, 0, 1)]
    for L in bad:
        lt = jas._launch(L)
        assert fwd(d, launch=lt) == 7, L
    # rows over 16,384 keys always stream: one-pass geometries are refused
    dl = desc(B=1, H=1, S=4, N=20000)
    for L in [(1, 0, 0, 0), (4, 9, 0, 0), (0, 16, 0, 0)]:
        assert fwd(dl, launch=jas._launch(L)) == 7, L
    df = desc(B=1, H=1, S=4, N=20000, dtype=jas.JAS_DTYPE_F32)
    assert fwd(df, launch=jas._launch((0, 4, 0, 0))) == 7  # 4 is a 16-bit segment size


def test_binding_rejects_host_tensors():
    # the torch-level wrappers refuse tensors outside device memory before
    # any pointer reaches the library
    import torch
    s = torch.zeros((1, 1, 2, 256))
    with pytest.raises(ValueError, match="device memory"):
        jas.fwd(s)
    with pytest.raises(ValueError, match="device memory"):
        jas.bwd(s, s)
    # the autograd Function marshals into the same calls: no host fallback
    from deterministic_attention_softmax_amd.autograd import softmax
    x = s.clone().requires_grad_(True)
    with pytest.raises(ValueError, match="device memory"):
        softmax(x)


def adesc(B=1, H=4, Hkv=2, Sq=16, N=300, D=128, dtype=jas.JAS_DTYPE_BF16, flags=0):
    return jas.make_attn_desc(B, H, Hkv, Sq, N, D, dtype, flags, 0.125)


def attn(d, q=A, k=B_, v=C, out=D, mask=None, key_len=None, sink=None, lse=None, p_sink=None,
         probs=None, scores=None):
    return jas.jas_attn_fwd(d, q, k, v, mask, key_len, sink, out, lse, p_sink, probs, scores, None)


def test_noalloc_validation():
    # jas_bwd_noalloc: the checks of jas_bwd without the workspace, then the
    # row limit of the library's scratch with a sink; every call below is
    # refused before any HIP call
    def nb(d, probs=A, dprobs=B_, p_sink=None, dscores=C, d_sink=None, key_len=None):
        return jas.jas_bwd_noalloc(d, probs, dprobs, key_len, p_sink, dscores, d_sink, None)
    sink = jas.JAS_FLAG_SINK
    big = jas.JAS_NOALLOC_MAX_ROWS
    assert nb(desc(B=1, H=1, S=big + 1, N=64, flags=sink), p_sink=D, d_sink=E) == 10
    assert nb(desc(B=2, H=4, S=big // 8 + 1, N=64, flags=sink), p_sink=D, d_sink=E) == 10
    assert jas.jas_status_str(10) == \
        "more rows than the library's scratch holds (JAS_NOALLOC_MAX_ROWS)"
    assert nb(desc(flags=sink), p_sink=None, d_sink=E) == 1       # flag without its pointer
    assert nb(desc(flags=sink), p_sink=D, d_sink=None) == 1
    assert nb(desc(), p_sink=D) == 4                               # pointer without its flag
    assert nb(desc(flags=sink), probs=None, p_sink=D, d_sink=E) == 1
    assert nb(desc(flags=sink), dscores=A, dprobs=A + 2, p_sink=D, d_sink=E) == 5
    assert nb(desc(N=jas.JAS_MAX_KEYS + 1, flags=sink), p_sink=D, d_sink=E) == 7
    assert jas.lib().jas_bwd_noalloc(None, A, B_, None, None, C, None, None) == 1


def test_attention_validation():
    # every call fails validation: a call that passed would launch on fake addresses
    assert attn(adesc(dtype=jas.JAS_DTYPE_F32)) == 3
    assert attn(adesc(D=96)) == 7
    assert attn(adesc(N=jas.JAS_ATTN_MAX_KEYS + 1)) == 7
    assert attn(adesc(H=3, Hkv=2)) == 2
    assert attn(adesc(N=0)) == 2
    # one (batch, head)'s mask must end within 2 GiB: 40,000 query rows of
    # 16,384 keys do not
    big = adesc(Sq=40000, N=16384, flags=jas.JAS_FLAG_MASK)
    big.mask_stride_q = 16384
    assert attn(big, mask=W) == 7
    assert attn(adesc(flags=1 << 7)) == 4
    assert attn(adesc(), mask=W) == 4                     # pointer without its flag
    assert attn(adesc(), probs=W) == 4
    assert attn(adesc(flags=jas.JAS_FLAG_LSE)) == 1       # flag without its pointer
    assert attn(adesc(flags=jas.JAS_FLAG_SCORES)) == 1
    assert attn(adesc(), q=None) == 1
    assert attn(adesc(), q=A + 8) == 9                    # 16-byte alignment of q, k, v
    assert attn(adesc(), out=A) == 5                      # out over q
    assert attn(adesc(flags=jas.JAS_FLAG_LSE), lse=D + 4) == 5   # lse inside out
    L = jas.lib()
    assert L.jas_attn_fwd(None, A, B_, C, None, None, None, D, None, None, None, None, None) == 1
    # jas_attn_fwd_ex: 16-query blocks per wavefront 0, 1 or 2; anything else
    # is refused before a pointer is looked at
    for qb in (-1, 3, 64):
        assert jas.jas_attn_fwd_ex(adesc(), A, B_, C, None, None, None, D, None, None, None, None,
                                   qb, None) == 4
    assert jas.jas_attn_fwd_ex(adesc(dtype=jas.JAS_DTYPE_F32), A, B_, C, None, None, None, D, None,
                               None, None, None, 2, None) == 3
    assert jas.jas_attn_fwd_ex(adesc(), None, B_, C, None, None, None, D, None, None, None, None,
                               2, None) == 1


def test_streaming_workgroup_sizes():
    # streaming: 4 waves, or 8 for 16-bit types (the larger segment only);
    # the default takes 8 for the 16-bit backward on rows of whole chunks up
    # to 65,536 keys, 4 for the forward
    L = jas.jas_launch_t
    for dt, wide_ok in ((jas.JAS_DTYPE_BF16, True), (jas.JAS_DTYPE_F16, True), (jas.JAS_DTYPE_F32, False)):
        d = desc(N=40000, dtype=dt)
        cpl = 16 if dt == jas.JAS_DTYPE_F32 else 8
        st, p = jas.jas_launch_plan(d, 0, L(8, cpl, 1, 0, 1))
        assert (st == 0) == wide_ok, (dt, st)
        st, p = jas.jas_launch_plan(d, 1, L(8, cpl // 2, 1, 0, 1))
        assert st == 7, (dt, st)                         # the wide workgroup: larger segment only
        assert jas.jas_launch_plan(d, 0, L(16, cpl, 1, 0, 1))[0] == 7
        st, p = jas.jas_launch_plan(d, 1)
        assert st == 0 and p.streaming == 1 and p.waves_per_row == (8 if wide_ok else 4)
        st, p = jas.jas_launch_plan(d, 0)
        assert st == 0 and p.streaming == 1 and p.waves_per_row == 4
    st, p = jas.jas_launch_plan(desc(N=65536), 1)
    assert p.waves_per_row == 8
    st, p = jas.jas_launch_plan(desc(N=65544), 1)
    assert p.waves_per_row == 4                          # more than two wide segments
    st, p = jas.jas_launch_plan(desc(N=40001), 1)
    assert p.waves_per_row == 4                          # not whole 16-byte chunks
    # the wide backward takes two rows per workgroup from 2,048 rows, unless
    # a geometry is given; the forward and the 4-wave backward one each
    big = desc(B=1, H=16, S=512, N=65536)
    st, p = jas.jas_launch_plan(big, 1)
    assert st == 0 and (p.waves_per_row, p.max_blocks) == (8, 4096)
    st, p = jas.jas_launch_plan(big, 0)
    assert st == 0 and (p.waves_per_row, p.max_blocks) == (4, 8192)
    st, p = jas.jas_launch_plan(big, 1, jas._launch((8, 8, 1, 0, 1)))
    assert st == 0 and p.max_blocks == 8192
    st, p = jas.jas_launch_plan(desc(B=1, H=16, S=127, N=65536), 1)
    assert st == 0 and p.max_blocks == 16 * 127          # fewer than 2,048 rows
    st, p = jas.jas_launch_plan(desc(B=1, H=16, S=512, N=65544), 1)
    assert st == 0 and (p.waves_per_row, p.max_blocks) == (4, 8192)


def _plan_covers(d, backward):
    st, p = jas.jas_launch_plan(d, backward)
    assert st == 0, (d.keys, d.dtype, backward, jas.STATUS.get(st, st))
    if p.streaming:
        assert d.keys > 16384 and p.rows_per_block == 1
        wide = (backward and d.dtype != jas.JAS_DTYPE_F32 and d.keys <= 65536 and d.keys % 8 == 0)
        assert p.waves_per_row == (8 if wide else 4), (d.keys, d.dtype, p.waves_per_row)
        return p
    kps = 256 if d.dtype == jas.JAS_DTYPE_F32 else 512          # keys per 64-lane slot
    assert p.waves_per_row in (1, 2, 4) and p.waves_per_row * p.rows_per_block <= 4
    assert p.waves_per_row * p.chunks_per_lane * kps >= d.keys, (d.keys, d.dtype, p.waves_per_row,
                                                                 p.chunks_per_lane)
    return p


@pytest.mark.parametrize("dtype", [jas.JAS_DTYPE_F32, jas.JAS_DTYPE_BF16, jas.JAS_DTYPE_F16])
def test_default_geometry_exists_for_every_row_length(dtype):
    # every row length up to the one-pass limit, and a sample beyond it, gets
    # a default geometry that holds the row, forward and backward (an fp32
    # row of 4,353 to 4,608 keys once had none)
    for N in list(range(1, 16385)) + [16385, 20000, 65536, 262143, 262144]:
        for backward in (0, 1):
            _plan_covers(desc(B=1, H=1, S=1, N=N, dtype=dtype), backward)
    st, _ = jas.jas_launch_plan(desc(N=262145, dtype=dtype), 0)
    assert jas.STATUS.get(st) == "JAS_ERR_UNSUPPORTED"


def test_mask_in_registers_choice():
    # The forward keeps the mask row in registers by default only where
    # consecutive rows share it: a mask broadcast over queries, no causal
    # flag, 16-bit 16-byte rows on two waves with at most 5 chunks per lane,
    # and at least 16,384 rows.  Then one row per workgroup and half as many
    # workgroups as rows.
    U = "JAS_ERR_UNSUPPORTED"
    M, CAUSAL = jas.JAS_FLAG_MASK, jas.JAS_FLAG_CAUSAL
    joint = dict(B=1, H=24, S=4352, N=4352, flags=M, ms=(4352, 0, 0))
    rows = 24 * 4352
    st, p = jas.jas_launch_plan(desc(**joint), 0)
    assert st == 0 and p.mask_in_registers == 1
    assert (p.waves_per_row, p.chunks_per_lane, p.rows_per_block) == (2, 5, 1)
    assert p.max_blocks == rows // 2 and p.streaming == 0
    # not by default: backward, a mask varying by query, the causal flag,
    # fp32, no mask, too few rows, rows not whole chunks, a geometry given
    for d, bw in [(desc(**joint), 1),
                  (desc(**{**joint, "ms": (4352 * 4352, 0, 4352)}), 0),
                  (desc(**{**joint, "flags": M | CAUSAL}), 0),
                  (desc(**{**joint, "dtype": jas.JAS_DTYPE_F32}), 0),
                  (desc(**{**joint, "flags": 0}), 0),
                  (desc(**{**joint, "S": 600}), 0),
                  (desc(**{**joint, "N": 4351, "ms": (4351, 0, 0)}), 0)]:
        st, p = jas.jas_launch_plan(d, bw)
        assert st == 0 and p.mask_in_registers == 0, (d.flags, d.keys, d.dtype, bw)
    st, p = jas.jas_launch_plan(desc(**joint), 0, jas._launch((2, 5, 0, 0, 0)))
    assert st == 0 and p.mask_in_registers == 0 and p.rows_per_block == 2
    st, p = jas.jas_launch_plan(desc(**joint), 0, jas._launch((0, 0, 0, 0, 0, 2)))
    assert st == 0 and p.mask_in_registers == 0 and p.max_blocks == rows // 2
    # asked for: any mask, any row count; the geometry fields still apply
    small = desc(B=2, H=3, S=5, N=4352, flags=M, ms=(4352, 0, 4352))
    st, p = jas.jas_launch_plan(small, 0, jas._launch((0, 0, 0, 0, 0, 1)))
    assert st == 0 and p.mask_in_registers == 1
    assert (p.rows_per_block, p.max_blocks) == (1, 15)
    st, p = jas.jas_launch_plan(small, 0, jas._launch((2, 5, 2, 7, 0, 1)))
    assert st == 0 and p.mask_in_registers == 1 and (p.rows_per_block, p.max_blocks) == (2, 7)
    # rows that are not whole 16-byte chunks: asked for, it runs (the element-wise forward)
    st, p = jas.jas_launch_plan(desc(B=2, H=3, S=5, N=4351, flags=M, ms=(4351, 0, 0)), 0,
                                jas._launch((0, 0, 0, 0, 0, 1)))
    assert st == 0 and p.mask_in_registers == 1
    # rows the default gives one wave: asked for, it takes two (5 slots: 3 chunks each)
    st, p = jas.jas_launch_plan(desc(B=2, H=3, S=5, N=2560, flags=M, ms=(2560, 0, 0)), 0,
                                jas._launch((0, 0, 0, 0, 0, 1)))
    assert st == 0 and p.mask_in_registers == 1 and (p.waves_per_row, p.chunks_per_lane) == (2, 3)
    # asked for where it is not built: an error, no plan
    for d, bw, ov in [(small, 1, (0, 0, 0, 0, 0, 1)),
                      (small, 0, (1, 9, 0, 0, 0, 1)),
                      (small, 0, (4, 3, 0, 0, 0, 1)),
                      (small, 0, (0, 0, 0, 0, 1, 1)),
                      (desc(B=2, H=3, S=5, N=4352), 0, (0, 0, 0, 0, 0, 1)),
                      (desc(B=2, H=3, S=5, N=4352, flags=M, dtype=jas.JAS_DTYPE_F32), 0,
                       (0, 0, 0, 0, 0, 1)),
                      (small, 0, (0, 0, 0, 0, 0, 3)),
                      (small, 0, (0, 0, 0, 0, 0, -1))]:
        st, p = jas.jas_launch_plan(d, bw, jas._launch(ov))
        assert jas.STATUS.get(st) == U and p.max_blocks == 0, (bw, ov)


def test_launch_plan_reports_overrides_and_errors():
    d = desc(B=2, H=3, S=5, N=1000, dtype=jas.JAS_DTYPE_BF16)
    st, p = jas.jas_launch_plan(d, 0, jas._launch((2, 1, 2, 0, 0)))
    assert st == 0 and (p.waves_per_row, p.chunks_per_lane, p.rows_per_block) == (2, 1, 2)
    assert p.max_blocks == (30 + 1) // 2 and p.streaming == 0
    st, p = jas.jas_launch_plan(d, 1, jas._launch((0, 0, 0, 4, 1)))   # 16-bit backward: wide
    assert st == 0 and p.streaming == 1 and p.max_blocks == 4 and p.waves_per_row == 8
    st, p = jas.jas_launch_plan(d, 0, jas._launch((0, 0, 0, 4, 1)))   # the forward: 4 waves
    assert st == 0 and p.streaming == 1 and p.waves_per_row == 4
    st, p = jas.jas_launch_plan(d, 1, jas._launch((4, 0, 0, 4, 1)))
    assert st == 0 and p.streaming == 1 and p.waves_per_row == 4
    st, p = jas.jas_launch_plan(d, 0, jas._launch((1, 1, 0, 0, 0)))   # 1 x 1 slot < 1000 keys
    assert jas.STATUS.get(st) == "JAS_ERR_UNSUPPORTED"
    assert (p.waves_per_row, p.chunks_per_lane, p.max_blocks) == (0, 0, 0)
    st, p = jas.jas_launch_plan(d, 2)
    assert jas.STATUS.get(st) == "JAS_ERR_BAD_FLAGS"
    st, p = jas.jas_launch_plan(desc(B=0), 0)                          # no rows: no launch
    assert st == 0 and p.max_blocks == 0
    assert jas.lib().jas_launch_plan(ctypes.byref(d), 0, None, None) == 1
