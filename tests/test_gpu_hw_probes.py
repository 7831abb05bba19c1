"""Exhaustive probes of the gfx950 instructions the library's arithmetic
rests on (test-only kernels in tests/hw_probes/):

* v_exp_f32 over every binary32 u from -0 down to -inf: its largest error
  against 2^u rounded to binary32, and that it returns +0 exactly where the
  exponential contract flushes (every u below -126) and a normal number from
  -126 up -- the kernels' exp_ relies on this instead of a select.
* v_cvt_pk_bf16_f32 over all 2^32 bit patterns: round to nearest-even, as the
  oracle's conversion (RL-Kernel PR #453: one dtype conversion at the write).
* the packed binary32 -> binary16 conversion over all 2^32 bit patterns: round
  to nearest-even with subnormals kept (RL-Kernel PR #240 lists FP16).
* v_log_f32 over every binary32 in [1, 32768] (the range of a row's sum of
  exponentials), the logarithm behind the row log-sum-exp: its largest error.
* the lane layout of the permlane16/32 swaps used by the tile trees.
* the operand and result layout of the 16x16x32 bf16 / fp16 MFMA the
  attention kernel uses.
"""
import ctypes
import os

import numpy as np
import pytest
import torch

from tests.gpu_util import log

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(__file__), "hw_probes", "libjas_hw_probes.so")


def probes():
    L = ctypes.CDLL(LIB)
    L.probe_exp2_sweep.restype = ctypes.c_int
    L.probe_exp2_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint32]
    L.probe_bf16_sweep.restype = ctypes.c_int
    L.probe_bf16_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32]
    L.probe_f16_sweep.restype = ctypes.c_int
    L.probe_f16_sweep.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint32]
    L.probe_log2_sweep.restype = ctypes.c_int
    L.probe_log2_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint32]
    L.probe_mfma_layout.restype = ctypes.c_int
    L.probe_mfma_layout.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    L.probe_permlane_layout.restype = ctypes.c_int
    L.probe_permlane_layout.argtypes = [ctypes.c_void_p]
    L.probe_tr16_layout.restype = ctypes.c_int
    L.probe_tr16_layout.argtypes = [ctypes.POINTER(ctypes.c_int), ctypes.c_void_p]
    return L


def test_v_exp_f32_sweep():
    L = probes()
    first = 0x80000000                     # -0.0
    last = 0xFF800000                      # -inf: every negative binary32
    count = last - first + 1
    words = 4 * ((count + 256 * 64 - 1) // (256 * 64))
    out = torch.zeros(words, dtype=torch.int32, device="cuda")
    nb = L.probe_exp2_sweep(first, count, out.data_ptr(), words)
    assert nb > 0
    r = out.cpu().numpy().view(np.uint32).reshape(-1, 4)
    max_ulp, ndiff, nlow, nnz = int(r[:, 0].max()), int(r[:, 1].sum()), int(r[:, 2].sum()), int(r[:, 3].sum())
    log(f"v_exp_f32 over {count} inputs in [-inf,0]: max {max_ulp} ulp, {ndiff} differ, "
        f"{nlow} below 2^-126 for u >= -126, {nnz} nonzero for u < -126")
    assert max_ulp <= 1
    assert nlow == 0 and nnz == 0


def test_v_cvt_pk_bf16_f32_is_rne_on_all_patterns():
    L = probes()
    count = 1 << 32
    words = 2 * (count // (256 * 64))
    out = torch.zeros(words, dtype=torch.int32, device="cuda")
    assert L.probe_bf16_sweep(0, count, out.data_ptr(), words) > 0
    r = out.cpu().numpy().view(np.uint32).reshape(-1, 2)
    bad, badnan = int(r[:, 0].sum()), int(r[:, 1].sum())
    log(f"v_cvt_pk_bf16_f32: {bad} non-NaN mismatches, {badnan} NaN results not NaN")
    assert bad == 0 and badnan == 0


def test_f16_conversion_is_rne_on_all_patterns():
    L = probes()
    count = 1 << 32
    words = 2 * (count // (256 * 64))
    out = torch.zeros(words, dtype=torch.int32, device="cuda")
    assert L.probe_f16_sweep(0, count, out.data_ptr(), words) > 0
    r = out.cpu().numpy().view(np.uint32).reshape(-1, 2)
    bad, badnan = int(r[:, 0].sum()), int(r[:, 1].sum())
    log(f"binary32 -> binary16: {bad} non-NaN mismatches, {badnan} NaN results not NaN")
    assert bad == 0 and badnan == 0


def test_v_log_f32_on_row_sum_range():
    # a row's L lies in [1, N + 1]: the largest key adds exactly 1, every
    # other term at most 1, the sink one more; N reaches 262,144 keys
    L = probes()
    first = int(np.float32(1.0).view(np.uint32))
    last = int(np.float32(2 ** 18 + 1).view(np.uint32))   # exact in binary32
    count = last - first + 1
    words = 2 * ((count + 256 * 64 - 1) // (256 * 64))
    out = torch.zeros(words, dtype=torch.int32, device="cuda")
    assert L.probe_log2_sweep(first, count, out.data_ptr(), words) > 0
    r = out.cpu().numpy().view(np.uint32).reshape(-1, 2)
    mx, nd = int(r[:, 0].max()), int(r[:, 1].sum())
    log(f"v_log_f32 on [1, 262145]: max {mx} ulp, {nd} of {count} differ from log2 rounded")
    assert mx <= 2


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_mfma_16x16x32_layout(dt):
    L = probes()
    g = torch.Generator().manual_seed(21)
    A = torch.randint(-4, 5, (16, 32), generator=g).to(dt)
    B = torch.randint(-4, 5, (32, 16), generator=g).to(dt)
    want = A.double() @ B.double()       # small integers: exact in fp32
    Ad = A.contiguous().view(torch.int16).to("cuda")
    Bd = B.contiguous().view(torch.int16).to("cuda")
    D = torch.zeros(256, dtype=torch.float32, device="cuda")
    assert L.probe_mfma_layout(Ad.data_ptr(), Bd.data_ptr(), D.data_ptr(),
                               int(dt == torch.float16)) == 0
    got = D.cpu().double().view(16, 16)
    log(f"mfma 16x16x32 {dt}: max |diff| {float((got - want).abs().max())}")
    assert torch.equal(got, want)


def test_permlane_swap_layout():
    L = probes()
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    assert L.probe_permlane_layout(out.data_ptr()) == 0
    r = out.cpu().numpy().reshape(64, 4)
    lanes = np.arange(64)
    # every lane sees (its even 16-lane row's value, the odd row's value) of
    # its 32-lane half, and (lower half's value, upper half's value)
    row_even = (lanes // 32) * 32 + (lanes % 16)
    assert np.array_equal(r[:, 0], row_even) and np.array_equal(r[:, 1], row_even + 16)
    assert np.array_equal(r[:, 2], lanes % 32) and np.array_equal(r[:, 3], lanes % 32 + 32)


def test_ds_read_b64_tr_b16_layout():
    # the fused attention builds its PV operand with this read: in each group
    # of 16 lanes the 16 addressed 8-byte chunks form a 16 x 4 matrix C
    # (C[j][p] = element p of lane j's chunk), and lane i receives
    # C[4e + i/4][i % 4] for e = 0..3
    L = probes()
    VROW = 144  # the kernel's V row (head dim 128 + 16), elements

    def vrow(r):
        return r ^ (((r >> 3) & 1) << 2)

    patterns = {"consecutive chunks": [4 * l for l in range(64)]}
    for db, half in ((0, 0), (3, 1), (7, 0)):
        patterns[f"attention V operand db={db} keys +{4 * half}"] = [
            vrow(8 * (l // 16) + 4 * half + (l % 16) // 4) * VROW + 16 * db + 4 * (l % 4)
            for l in range(64)]
    for name, addr in patterns.items():
        out = torch.zeros(256, dtype=torch.int16, device="cuda")
        arr = (ctypes.c_int * 64)(*addr)
        assert L.probe_tr16_layout(arr, out.data_ptr()) == 0, name
        got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
        want = np.zeros((64, 4), np.int64)
        for l in range(64):
            g, i = l // 16, l % 16
            for e in range(4):
                want[l, e] = addr[16 * g + 4 * e + i // 4] + i % 4
        log(f"ds_read_b64_tr_b16, {name}: {int((got != want).sum())} mismatches")
        assert np.array_equal(got, want), name
    # the attention operand: lane (g, c16) gets dim 16*db + c16 of keys
    # 8g + 4*half .. +3, in key order
    addr = patterns["attention V operand db=3 keys +4"]
    out = torch.zeros(256, dtype=torch.int16, device="cuda")
    assert L.probe_tr16_layout((ctypes.c_int * 64)(*addr), out.data_ptr()) == 0
    got = out.cpu().numpy().astype(np.int64).reshape(64, 4)
    for l in range(64):
        g, c16 = l // 16, l % 16
        assert [int(v) for v in got[l]] == [vrow(8 * g + 4 + e) * VROW + 48 + c16 for e in range(4)]
