"""Pins for the oracle's MoE dispatch / combine (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import bf16, moe
from reduce_rank_buffers_amd import inputs
from tests import _exact


def _routing(T, E, k, seed):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    return idx, w


def _tokens(T, h, R, seed):
    rng = np.random.default_rng(seed)
    x = bf16.rne(rng.standard_normal(T * h).astype(np.float32)).reshape(T, h)
    return [x[r * (T // R):(r + 1) * (T // R)] for r in range(R)], x


@pytest.mark.parametrize("T,E,k,R", [(16, 8, 2, 4), (64, 32, 4, 8), (40, 16, 8, 8)])
def test_dispatch_invariants(T, E, k, R):
    idx, _ = _routing(T, E, k, T + E)
    shards, x = _tokens(T, 5, R, 1)
    recv = moe.dispatch(shards, idx, E)
    toks, counts, offsets, rows = moe.layout(idx, E, R)
    assert counts.sum() == T * k
    assert sum(r.shape[0] for r in recv) == T * k
    per = E // R
    for e in range(E):
        r = e // per
        ts = toks[e]
        assert all(a < b for a, b in zip(ts, ts[1:]))  # strictly ascending tokens
        for i, t in enumerate(ts):
            assert np.array_equal(recv[r][offsets[e] + i], x[t])
        # offsets are the exclusive prefix over the rank's experts
        first = r * per
        assert offsets[e] == counts[first:e].sum()


def test_dispatch_gather_back_reproduces_tokens():
    T, E, k, R = 64, 32, 4, 8
    idx, _ = _routing(T, E, k, 2)
    shards, x = _tokens(T, 7, R, 3)
    recv = moe.dispatch(shards, idx, E)
    toks, counts, offsets, rows = moe.layout(idx, E, R)
    per = E // R
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            i = toks[e].index(t)
            assert np.array_equal(recv[e // per][offsets[e] + i], x[t])


def test_combine_one_hot_weights_select_one_slot():
    T, E, k, R, h = 32, 16, 4, 4, 6
    idx, _ = _routing(T, E, k, 4)
    w = np.zeros((T, k), dtype=np.float32)
    pick = np.random.default_rng(5).integers(0, k, size=T)
    w[np.arange(T), pick] = 1.0
    toks, counts, offsets, rows = moe.layout(idx, E, R)
    z = [bf16.rne(np.random.default_rng(6 + r).standard_normal((int(n), h)).astype(np.float32))
         for r, n in enumerate(rows)]
    y = np.concatenate(moe.combine(z, idx, w, E, T // R))
    per = E // R
    for t in range(T):
        e = int(idx[t, pick[t]])
        zz = z[e // per][offsets[e] + toks[e].index(t)]
        # w*z with w=1 is exact; adding +0 terms keeps it (unless z = -0)
        want = np.where(zz == 0x8000, 0x0000, zz)
        assert np.array_equal(y[t], want)


def test_combine_exact_emulation_tiny():
    T, E, k, R, h = 16, 8, 4, 4, 5
    idx, w = _routing(T, E, k, 7)
    toks, counts, offsets, rows = moe.layout(idx, E, R)
    z = [bf16.rne(np.random.default_rng(8 + r).standard_normal((int(n), h)).astype(np.float32))
         for r, n in enumerate(rows)]
    y = np.concatenate(moe.combine(z, idx, w, E, T // R))
    per = E // R
    for t in range(T):
        pairs = sorted((int(idx[t, j]), float(w[t, j])) for j in range(k))
        for col in range(h):
            acc = None
            for e, wt in pairs:
                zv = _exact.bf16_value(int(z[e // per][offsets[e] + toks[e].index(t)][col]))
                term = _exact.f32_mul(wt, zv)
                acc = term if acc is None else _exact.f32_add(acc, term)
            assert int(y[t, col]) == _exact.to_bf16_bits(acc)


def test_combine_uses_ascending_expert_order_not_topk_order():
    # A token whose top-k order differs from ascending id: the fp32 rounding
    # of 2^24 + 1 makes the order visible.
    idx = np.array([[3, 1, 2, 0]], dtype=np.int32)
    w = np.ones((1, 4), dtype=np.float32)
    vals = {0: 2.0 ** 24, 1: 1.0, 2: -(2.0 ** 24), 3: 0.0}
    # one expert per rank with R = 4, E = 4: rank e holds expert e
    z = [bf16.rne(np.array([[vals[e]]], dtype=np.float32)) for e in range(4)]
    # T = 4 tokens (one per rank) all routed the same way
    idx4 = np.repeat(idx, 4, axis=0)
    w4 = np.repeat(w, 4, axis=0)
    z4 = [np.repeat(x, 4, axis=0) for x in z]
    y = np.concatenate(moe.combine(z4, idx4, w4, 4, 1))
    # ascending id: 2^24 + 1 rounds to 2^24 (tie, even), - 2^24 = 0, + 0 = 0;
    # the top-k order 3, 1, 2, 0 would give 0 + 1 - 2^24 + 2^24 = 1 (0x3F80)
    assert np.all(y[:, 0] == 0x0000)


# An fp32 weight whose exact product with 5.0 is 2^-8 + 2^-24 + 2^-33: one
# binary32 multiply rounds it to 2^-8 + 2^-24, and 1 + that is an fp32 tie
# that goes to 1 + 2^-8, itself a bf16 tie that goes to 1.0.  A fused
# multiply-add keeps the 2^-33 and lands on 1 + 2^-7 instead.
FMA_W_BITS = 978111898
FMA_Z = 5.0


def test_fma_case_premises_hold_exactly():
    w = float(np.array([FMA_W_BITS], dtype=np.uint32).view(np.float32)[0])
    prod = Fraction(w) * Fraction(FMA_Z)
    assert prod == Fraction(1, 2 ** 8) + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 33)
    assert _exact.f32_mul(w, FMA_Z) == 2.0 ** -8 + 2.0 ** -24
    sep = _exact.f32_add(1.0, _exact.f32_mul(w, FMA_Z))
    fused = _exact.round_binary(Fraction(1) + prod, 24)
    assert _exact.to_bf16_bits(sep) == 0x3F80 and _exact.to_bf16_bits(fused) == 0x3F81


def test_combine_rounds_the_product_before_the_add():
    w1 = np.array([FMA_W_BITS], dtype=np.uint32).view(np.float32)[0]
    # R = 1, E = 2 (rank 0 holds both experts); one token, experts 1 then 0
    idx = np.array([[1, 0]], dtype=np.int32)
    w = np.array([[w1, 1.0]], dtype=np.float32)
    z = [bf16.rne(np.array([[1.0], [FMA_Z]], dtype=np.float32))]
    y = moe.combine(z, idx, w, 2, 1)
    # ascending id: expert 0 (z = 1.0, w = 1) then expert 1 (z = 5, w = w1)
    assert int(y[0][0, 0]) == 0x3F80


def test_gate_routing_is_valid():
    idx, w = inputs.moe_routing(T=256, E=256, k=8)
    assert idx.shape == (256, 8) and w.shape == (256, 8)
    for t in range(256):
        assert len(set(idx[t].tolist())) == 8
        assert np.all(np.diff(w[t]) <= 0)  # descending probabilities
    assert np.all(w > 0) and np.all(w.sum(axis=1) < 1.0 + 1e-6)
