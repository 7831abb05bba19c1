"""Pins for the oracle's scalar pieces: the exponential and bf16 rounding.

exp_: RL-Kernel PR #453 says all backends share one exponential approximation
without naming it; the reading is exp(y) = 2^(fl(y*log2e)), flushed below
2^-126.  Pinned against float64 exp with an error bound derived from the two
binary32 roundings.  bf16 rounding (one conversion at the write, same page)
is pinned against torch's CPU conversion, a library round-to-nearest-even.
"""
import math

import numpy as np
import pytest

import oracle as O
from tests.ref64 import U, f32_to_bf16_bits_torch


def test_log2e_is_nearest_binary32():
    L = O.log2e()
    exact = 1.0 / math.log(2.0)
    lo = np.nextafter(L, np.float32(0))
    hi = np.nextafter(L, np.float32(4))
    assert abs(float(L) - exact) < abs(float(lo) - exact)
    assert abs(float(L) - exact) < abs(float(hi) - exact)


def test_exp_special_values():
    assert O.exp_(0.0) == np.float32(1.0)
    assert O.exp_(-0.0) == np.float32(1.0)
    assert O.exp_(-np.inf) == np.float32(0.0)
    assert not np.signbit(O.exp_(-np.inf))


def test_exp_flush_boundary():
    L = O.log2e()
    # scan binary32 y around -126/log2e: exp_ is 2^-126 where fl(y*L) == -126
    # and +0 wherever fl(y*L) < -126
    y0 = np.array([-126.0 / float(L)], np.float32).view(np.int32)[0]
    ys = (y0 + np.arange(-40, 41, dtype=np.int32)).view(np.float32)
    seen_exact = seen_below = False
    for y in ys:
        u = np.float32(y * L)
        got = O.exp_(y)
        if u == np.float32(-126.0):
            assert got == np.float32(2.0 ** -126)
            seen_exact = True
        elif u < -126.0:
            assert got == 0.0
            seen_below = True
        else:
            assert got > np.float32(2.0 ** -126)
    assert seen_exact and seen_below
    assert O.exp_(-200.0) == np.float32(0.0)


def test_exp_error_bound_against_float64():
    # u = y*log2e*(1+e0)(1+e1), |e1| <= 2^-24, e0 = log2e_f32/log2e - 1;
    # 2^u = e^y * exp(y*(e0+e1+e0*e1)), then one rounding to binary32.
    L = O.log2e()
    e0 = abs(float(L) * math.log(2.0) - 1.0)
    rng = np.random.default_rng(11)
    ys = np.concatenate([
        -rng.exponential(3.0, 3000), -rng.uniform(0, 87.3, 3000),
        -rng.uniform(0, 1e-3, 500), np.array([-1e-30, -1e-7, -0.5, -1.0, -10.0, -80.0]),
    ]).astype(np.float32)
    for y in ys:
        got = float(O.exp_(y))
        u = float(np.float32(y * L))
        if u < -126.0:
            assert got == 0.0
            continue
        ref = math.exp(float(y))
        bound = U + abs(float(y)) * (e0 + U) * 1.001 + 1e-15
        assert abs(got - ref) <= bound * ref, (y, got, ref)


def test_exp_integer_powers_exact():
    # 2^k is exact in binary32, so an argument whose product rounds to an
    # integer must give exactly that power of two.
    L = O.log2e()
    for k in range(0, 127):
        y = np.float32(-k / float(L))
        if np.float32(y * L) == np.float32(-k):
            assert O.exp_(y) == np.float32(2.0 ** -k)


def _bf16_cases():
    rng = np.random.default_rng(5)
    rnd = rng.integers(0, 2 ** 32, 60000, dtype=np.uint64).astype(np.uint32)
    # ties (low 16 bits exactly 0x8000) with odd and even kept parts, and
    # neighbours of ties
    base = rng.integers(0, 2 ** 16, 4000, dtype=np.uint64).astype(np.uint32) << 16
    ties = np.concatenate([base | 0x8000, base | 0x7FFF, base | 0x8001, base])
    special = np.array([0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x7F7FFFFF,
                        0xFF7FFFFF, 0x7F7F8000, 0x00000001, 0x00008000, 0x00018000,
                        0x007FFFFF, 0x00800000, 0x3F808000, 0x3F818000, 0x3F7FFFFF],
                       dtype=np.uint32)
    bits = np.concatenate([rnd, ties, special])
    x = bits.view(np.float32)
    return x[~np.isnan(x)]


def test_bf16_rne_matches_torch():
    x = _bf16_cases()
    want = f32_to_bf16_bits_torch(x)
    got = np.array([O.bf16_rne(v) for v in x], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(x[i:i+1].view(np.uint32)[0]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_bf16_rne_nan_stays_nan():
    for bits in (0x7FC00000, 0x7F800001, 0xFFC00001, 0x7FFFFFFF):
        x = np.array([bits], np.uint32).view(np.float32)[0]
        h = O.bf16_rne(x)
        assert (h & 0x7F80) == 0x7F80 and (h & 0x7F) != 0
        assert (h >> 15) == (bits >> 31)


@pytest.mark.parametrize("v,expect", [(1.0, 0x3F80), (-2.0, 0xC000), (2.0 ** -133, 0x0001),
                                      (1.0 + 2.0 ** -8, 0x3F80), (1.0 + 3 * 2.0 ** -8, 0x3F82)])
def test_bf16_rne_worked_values(v, expect):
    # 1 + 2^-8 is half-way between 1 and 1 + 2^-7 (kept part even -> 1);
    # 1 + 3*2^-8 is half-way between 1 + 2^-7 and 1 + 2^-6 (odd -> up);
    # 2^-133 is the smallest bf16 subnormal.
    assert O.bf16_rne(v) == expect
