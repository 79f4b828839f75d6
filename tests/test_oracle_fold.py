"""Pins for the oracle's fixed-order fp32 fold (CPU only).

Against an exact rational emulation of binary32 addition (tests/_exact.py) on
tiny inputs with cancellation, overflow, subnormals and signed zeros; closed
forms; and the recursive-summation error bound on random data.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, fold
from tests import _exact


def _bits(vals):
    return bf16.rne(np.asarray(vals, dtype=np.float32))


SPECIAL = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80,
                    0x7F7F, 0xFF7F, 0x7F00, 0x4000, 0xC000, 0x3F81, 0xBF81, 0x0100],
                   dtype=np.uint16)


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8])
def test_fold_matches_exact_emulation_random(R):
    rng = np.random.default_rng(100 + R)
    n = 64
    ins = [rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16) for _ in range(R)]
    # keep finite inputs; infinities/NaN are outside the workloads
    ins = [np.where((x & 0x7F80) == 0x7F80, x & 0x3FFF, x).astype(np.uint16) for x in ins]
    got = fold.reduce_bf16(ins)
    for j in range(n):
        want = _exact.fold_bf16_exact([int(x[j]) for x in ins])
        assert int(got[j]) == want, (j, [hex(int(x[j])) for x in ins], hex(int(got[j])), hex(want))


@pytest.mark.parametrize("R", [2, 4, 8])
def test_fold_matches_exact_emulation_specials(R):
    rng = np.random.default_rng(200 + R)
    n = 256
    ins = [SPECIAL[rng.integers(0, len(SPECIAL), size=n)] for _ in range(R)]
    got = fold.reduce_bf16(ins)
    for j in range(n):
        want = _exact.fold_bf16_exact([int(x[j]) for x in ins])
        assert int(got[j]) == want, (j, [hex(int(x[j])) for x in ins])


def test_fold_order_matters_and_is_rank_order():
    # 2^24 + 1 - 2^24 style cancellation: order changes the fp32 result
    big = _bits([2.0 ** 24])[0]
    one = _bits([1.0])[0]
    nbig = _bits([-(2.0 ** 24)])[0]
    a = fold.reduce_bf16([np.array([big]), np.array([one]), np.array([nbig])])
    b = fold.reduce_bf16([np.array([big]), np.array([nbig]), np.array([one])])
    assert int(a[0]) == 0x0000          # (2^24 + 1) rounds to 2^24, then -2^24 -> +0
    assert int(b[0]) == int(one)        # 0 + 1 = 1


def test_closed_form_identity_R1():
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    x = x[(x & 0x7F80) != 0x7F80]
    assert np.array_equal(fold.reduce_bf16([x]), x)


@pytest.mark.parametrize("R", [2, 4, 8])
def test_closed_form_equal_ranks_power_of_two(R):
    rng = np.random.default_rng(5)
    x = _bits(rng.standard_normal(4096).astype(np.float32))
    got = fold.reduce_bf16([x] * R)
    want = _bits(bf16.widen(x) * np.float32(R))  # R*x is exact for R = 2^k
    assert np.array_equal(got, want)


def test_closed_form_cancelling_pairs():
    rng = np.random.default_rng(6)
    ins = []
    for _ in range(4):
        x = _bits(rng.standard_normal(1000).astype(np.float32))
        ins += [x, x ^ np.uint16(0x8000)]
    got = fold.reduce_bf16(ins)
    assert np.all(got == 0x0000)  # x + (-x) = +0 under round-to-nearest


def test_closed_form_small_integers():
    rng = np.random.default_rng(8)
    vals = rng.integers(-100, 100, size=(8, 500))
    got = fold.reduce_bf16([_bits(v.astype(np.float32)) for v in vals])
    want = _bits(vals.sum(axis=0).astype(np.float32))
    assert np.array_equal(got, want)


def test_negative_zero_fold_start():
    nz = np.array([0x8000], dtype=np.uint16)
    assert int(fold.reduce_bf16([nz] * 8)[0]) == 0x8000


def test_error_bound_random():
    rng = np.random.default_rng(9)
    R, n = 8, 300
    ins = [_bits(rng.standard_normal(n).astype(np.float32)) for _ in range(R)]
    s = fold.fold_f32([bf16.widen(x) for x in ins])
    u = Fraction(1, 1 << 24)
    gamma = (R - 1) * u / (1 - (R - 1) * u)
    for j in range(n):
        vals = [Fraction(float(bf16.widen(x[j:j + 1])[0])) for x in ins]
        exact = sum(vals)
        bound = gamma * sum(abs(v) for v in vals)
        assert abs(Fraction(float(s[j])) - exact) <= bound


def test_f32_fold_matches_exact_emulation():
    rng = np.random.default_rng(10)
    R, n = 8, 128
    ins = [rng.standard_normal(n).astype(np.float32) * np.float32(10.0 ** rng.integers(-30, 30))
           for _ in range(R)]
    got = fold.reduce_f32(ins)
    for j in range(n):
        s = float(ins[0][j])
        for x in ins[1:]:
            s = _exact.f32_add(s, float(x[j]))
        assert float(got[j]) == s or (np.isnan(got[j]) and np.isnan(s))
