"""Pins for the oracle's tree-order fold (CPU only).

The tree is a reading (pairwise, level by level, an odd last item passed up);
these tests fix it by hand-worked fp32 cases in which the association changes
the result, by an exact rational emulation of the same tree, by the pairwise
summation error bound, and by the tolerance the variant must keep against the
fixed-order fold.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, collectives as C, fold
from tests import _exact

B = float(2 ** 24)  # the first binary32 integer whose successor is not representable


def _f32(vals):
    return [np.array([v], dtype=np.float32) for v in vals]


# Hand-worked: with B = 2^24, B + 1 rounds to B (a tie, to the even B) while
# 1 - B = -(B - 1) is exact.
#   R=4 [B, 1, 1, -B]:            tree (B+1) + (1-B) = B - (B-1) = 1;       fixed 0
#   R=5 [B, 1, 1, -B, 1]:         tree 1 + 1 = 2;                            fixed 1
#   R=6 [B, 1, 1, -B, 1, 1]:      tree 1 + (1+1) = 3;                        fixed 2
#   R=7 [B, 1, 1, -B, 1, 1, 1]:   tree 1 + ((1+1)+1) = 4;                    fixed 3
#   R=8 [B, 1, 1, -B, B, 1, 1, -B]: tree ((B+1)+(1-B)) + ((B+1)+(1-B)) = 2;  fixed 0;
#       pairs folded left to right instead would give ((1 + B) + (1-B)) = 1.
HAND = [
    ([B, 1, 1, -B], 1.0, 0.0),
    ([B, 1, 1, -B, 1], 2.0, 1.0),
    ([B, 1, 1, -B, 1, 1], 3.0, 2.0),
    ([B, 1, 1, -B, 1, 1, 1], 4.0, 3.0),
    ([B, 1, 1, -B, B, 1, 1, -B], 2.0, 0.0),
]


@pytest.mark.parametrize("vals,tree,fixed", HAND)
def test_hand_worked_association(vals, tree, fixed):
    assert float(fold.fold_tree_f32(_f32(vals))[0]) == tree
    assert float(fold.fold_f32(_f32(vals))[0]) == fixed
    assert float(fold.reduce_tree(_f32(vals), "f32")[0]) == tree


@pytest.mark.parametrize("R", [1, 2, 3])
def test_small_R_equals_fixed_order(R):
    rng = np.random.default_rng(300 + R)
    ins = [rng.standard_normal(4096).astype(np.float32) * 1e3 for _ in range(R)]
    assert np.array_equal(fold.fold_tree_f32(ins).view(np.uint32), fold.fold_f32(ins).view(np.uint32))


def _tree_exact(vals):
    items = list(vals)
    while len(items) > 1:
        nxt = [_exact.f32_add(items[i], items[i + 1]) for i in range(0, len(items) - 1, 2)]
        if len(items) % 2:
            nxt.append(items[-1])
        items = nxt
    return items[0]


@pytest.mark.parametrize("R", [4, 5, 6, 7, 8, 11, 16])
def test_tree_matches_exact_emulation(R):
    rng = np.random.default_rng(400 + R)
    n = 48
    ins = [rng.integers(0, 1 << 16, size=n, dtype=np.uint32).astype(np.uint16) for _ in range(R)]
    ins = [np.where((x & 0x7F80) == 0x7F80, x & 0x3FFF, x).astype(np.uint16) for x in ins]
    got = fold.reduce_tree(ins, "bf16")
    for j in range(n):
        s = _tree_exact([_exact.bf16_value(int(x[j])) for x in ins])
        assert int(got[j]) == _exact.to_bf16_bits(s), (R, j)


@pytest.mark.parametrize("R", [4, 8, 16])
def test_pairwise_error_bound(R):
    """|tree - exact| <= ceil(log2 R) 2^-24 sum|x| before the bf16 rounding:
    every term passes through ceil(log2 R) additions."""
    rng = np.random.default_rng(500 + R)
    n = 256
    ins = [bf16.widen(bf16.rne(rng.standard_normal(n).astype(np.float32))) for _ in range(R)]
    t = fold.fold_tree_f32(ins)
    depth = math.ceil(math.log2(R))
    for j in range(n):
        exact = sum(Fraction(float(x[j])) for x in ins)
        mag = sum(abs(Fraction(float(x[j]))) for x in ins)
        assert abs(Fraction(float(t[j])) - exact) <= depth * Fraction(1, 2 ** 24) * mag


def ulp_bf16(y):
    a = np.abs(y.astype(np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _tree_vs_fixed(ins, R):
    fx = bf16.widen(fold.reduce_bf16(ins)).astype(np.float64)
    tr = bf16.widen(fold.reduce_tree(ins, "bf16")).astype(np.float64)
    mag = np.sum([np.abs(bf16.widen(x).astype(np.float64)) for x in ins], axis=0)
    tol = np.maximum(ulp_bf16(fx), 2 * (R - 1) * 2.0 ** -24 * mag)
    return fx, tr, tol


@pytest.mark.parametrize("R", [4, 8, 16])
def test_tolerance_against_fixed_order_wide_range(R):
    """The variant's bar: |tree - fixed| <= max(1 ulp_bf16(fixed),
    2 (R-1) 2^-24 sum|x|).  Terms spread over 2^-24 .. 2^24 so that the fp32
    partial sums round and the two orders really differ."""
    rng = np.random.default_rng(600 + R)
    n = 1 << 16
    ins = [bf16.rne((rng.standard_normal(n) * 2.0 ** rng.integers(-24, 25, n)).astype(np.float32))
           for _ in range(R)]
    fx, tr, tol = _tree_vs_fixed(ins, R)
    assert np.all(np.abs(tr - fx) <= tol)
    assert np.any(tr != fx)
    # The plain 1-ulp rule can fail under cancellation (reported, not required).
    over = int(np.sum(np.abs(tr - fx) > ulp_bf16(fx)))
    print(f"R={R}: {int(np.sum(tr != fx))} differ, {over} beyond 1 bf16 ulp")


@pytest.mark.parametrize("R", [4, 8, 16])
def test_orders_agree_almost_everywhere_on_unit_normal_data(R):
    """A bf16 term has an 8-bit significand, so an fp32 sum of at most 16 of
    them is exact unless the terms span more than about 2^12: on N(0, 1)
    data the two orders give the same bits almost everywhere."""
    rng = np.random.default_rng(700 + R)
    ins = [bf16.rne(rng.standard_normal(1 << 16).astype(np.float32)) for _ in range(R)]
    fx, tr, tol = _tree_vs_fixed(ins, R)
    assert np.all(np.abs(tr - fx) <= tol)
    assert np.all(np.abs(tr - fx) <= ulp_bf16(fx))  # the plain 1-ulp rule holds here
    assert np.mean(tr != fx) <= 1e-3


def test_collective_reduce_tree_is_all_reduce_in_tree_order():
    rng = np.random.default_rng(7)
    R, n = 8, 64
    ins = [bf16.rne(rng.standard_normal(n).astype(np.float32)) for _ in range(R)]
    outs = C.collective(C.PARTIAL, C.REPLICATED, "reduce_tree", ins, R, n)
    want = fold.reduce_tree(ins, "bf16")
    for o in outs:
        assert np.array_equal(o, want)
    rs = C.collective(C.PARTIAL, C.SHARD, "reduce_tree", ins, R, n)
    for q in range(R):
        assert np.array_equal(rs[q], want[q * (n // R):(q + 1) * (n // R)])
