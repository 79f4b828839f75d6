"""GPU parity of device-side MoE routing (maps built on the GPU from device
routing arrays) against the oracle, through the C ABI: the receive arena is
the concatenation of the oracle's per-rank receive buffers, rank offsets are
the running sums of its per-rank row counts, combine is bit-exact.  Also:
re-routing with new routing, bad routing reported and kept in bounds, and
agreement with the host-built row plan."""

import sys

import numpy as np
import pytest
import torch

from oracle import bf16, moe as OM
from reduce_rank_buffers_amd import _lib as L, api, inputs
from tests.gpu_util import DEV, assert_bits_equal, empty_like_np, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run(T, h, E, k, R, idx, w, x_shards, z_np=None):
    disp = api.MoeDevicePlan(R, T, h, E, k, "dispatch")
    comb = api.MoeDevicePlan(R, T, h, E, k, "combine", share=disp)
    d_idx = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to(DEV)
    d_w = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(DEV)
    offs = torch.zeros(R + 1, dtype=torch.int32, device=DEV)
    disp.route(d_idx, d_w, offs)
    xs = [to_dev(s.reshape(-1)) for s in x_shards]
    arena = empty_like_np(T * k * h, "bf16", -21555)
    disp.run(xs, [arena] + [None] * (R - 1))
    disp.check()
    want_recv = OM.dispatch(x_shards, idx, E)
    _, counts, offsets, rows = OM.layout(idx, E, R)
    want_offs = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    assert np.array_equal(offs.cpu().numpy(), want_offs)
    got = from_dev(arena).reshape(T * k, h)
    assert_bits_equal(got, np.concatenate(want_recv, axis=0), "device-routed dispatch arena")
    if z_np is None:
        z_np, z_arena = want_recv, arena
    else:
        z_arena = to_dev(np.concatenate(z_np, axis=0).reshape(-1))
    y = [empty_like_np(T // R * h, "bf16", -21555) for _ in range(R)]
    comb.run([z_arena] + [None] * (R - 1), y)
    torch.cuda.synchronize()
    want_y = OM.combine(z_np, idx, w, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want_y[r], f"device-routed combine rank {r}")
    return disp, comb


def test_device_routing_full_workload():
    require_gpu()
    _say("device routing: 4096 x 7168, 256 experts, top-8")
    T, h, E, k, R = 4096, 7168, 256, 8, 8
    idx, w = inputs.moe_routing(T, E, k)
    x = inputs.moe_tokens(T, h, R)
    _run(T, h, E, k, R, idx, w, x)


@pytest.mark.parametrize("T,h,E,k,R", [(104, 24, 16, 3, 8), (512, 16, 1024, 16, 8), (40, 8, 8, 1, 4),
                                       (8, 13, 4, 2, 2), (1000, 64, 64, 8, 8)])
def test_device_routing_shapes(T, h, E, k, R):
    require_gpu()
    rng = np.random.default_rng(T + E + k)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _, counts, offsets, rows = OM.layout(idx, E, R)
    z = [bf16.rne(rng.standard_normal((int(n), h)).astype(np.float32)) for n in rows]
    _run(T, h, E, k, R, idx, w, shards, z)


def test_device_rerouting_and_host_plan_agree():
    require_gpu()
    T, h, E, k, R = 1024, 128, 64, 4, 8
    rng = np.random.default_rng(5)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    disp = api.MoeDevicePlan(R, T, h, E, k, "dispatch")
    xs = [to_dev(s.reshape(-1)) for s in shards]
    for step in range(3):
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        if step == 2:
            idx[:, 0] = 7  # skewed: every token picks expert 7
            for t in range(T):
                row = [e for e in idx[t, 1:] if e != 7]
                while len(row) < k - 1:
                    c = int(rng.integers(E))
                    if c != 7 and c not in row:
                        row.append(c)
                idx[t, 1:] = row
        w = rng.random((T, k)).astype(np.float32)
        disp.route(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV))
        arena = empty_like_np(T * k * h, "bf16")
        disp.run(xs, [arena] + [None] * (R - 1))
        disp.check()
        host = api.MoePlan(R, h, E, idx, w, "dispatch")
        recv = [empty_like_np(r * h, "bf16") for r in host.rows_per_rank]
        host.run(xs, recv)
        torch.cuda.synchronize()
        cat = np.concatenate([from_dev(t) for t in recv])
        assert_bits_equal(from_dev(arena), cat, f"step {step}: device vs host row plan")


@pytest.mark.parametrize("T", [64, 4096, 262144])
def test_device_routing_bad_rows_write_nothing(T):
    """A routing with a repeated or out-of-range expert is reported by the
    check, and the dispatch and combine that follow write nothing: every
    receive row and every token output keeps its earlier contents (no valid
    row is overwritten).  A later valid routing works again.  T = 64 and 4096
    take the fused routing kernel, 262,144 tokens the three-kernel path."""
    require_gpu()
    h, E, k, R = 16, 16, 2, 4
    rng = np.random.default_rng(T)
    good = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    for bad_kind in ("repeat", "range"):
        idx = good.copy()
        if bad_kind == "repeat":
            idx[T // 3] = [5, 5]
        else:
            idx[T - 1] = [1, 99]
        w = rng.random((T, k)).astype(np.float32)
        disp = api.MoeDevicePlan(R, T, h, E, k, "dispatch")
        comb = api.MoeDevicePlan(R, T, h, E, k, "combine", share=disp)
        disp.route(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV))
        arena = empty_like_np(T * k * h, "bf16", -21555)
        y = [empty_like_np(T // R * h, "bf16", -21555) for _ in range(R)]
        xs = [empty_like_np(T // R * h, "bf16", 1) for _ in range(R)]
        disp.run(xs, [arena] + [None] * (R - 1))
        comb.run([arena] + [None] * (R - 1), y)
        with pytest.raises(L.RrbError) as e:
            disp.check()
        assert e.value.status == L.RRB_EINVAL, bad_kind
        assert np.all(from_dev(arena) == np.uint16(0xABCD)), f"{bad_kind}: dispatch wrote rows"
        for r in range(R):
            assert np.all(from_dev(y[r]) == np.uint16(0xABCD)), f"{bad_kind}: combine wrote rank {r}"
        # a valid routing on the same workspace clears the failure
        disp.route(torch.from_numpy(good).to(DEV), torch.from_numpy(w).to(DEV))
        disp.run(xs, [arena] + [None] * (R - 1))
        disp.check()
        shards = [np.ones((T // R, h), np.uint16) for _ in range(R)]
        want = np.concatenate(OM.dispatch(shards, good, E), axis=0)
        assert_bits_equal(from_dev(arena).reshape(T * k, h), want, f"{bad_kind}: re-routed dispatch")


def test_device_combine_per_call_weights():
    """rrb_reduce's per-call weights on a device-routed combine plan: weights
    given in the routing order replace the routed ones for that call only."""
    require_gpu()
    T, h, E, k, R = 512, 136, 32, 4, 8
    rng = np.random.default_rng(77)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    w2 = (rng.standard_normal((T, k)) * 3).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _, _, _, rows = OM.layout(idx, E, R)
    z = [bf16.rne(rng.standard_normal((int(n), h)).astype(np.float32)) for n in rows]
    disp, comb = _run(T, h, E, k, R, idx, w, shards, z)
    z_arena = to_dev(np.concatenate(z, axis=0).reshape(-1))
    y = [empty_like_np(T // R * h, "bf16", -21555) for _ in range(R)]
    comb.run([z_arena] + [None] * (R - 1), y, weights=torch.from_numpy(w2).to(DEV))
    torch.cuda.synchronize()
    want2 = OM.combine(z, idx, w2, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want2[r], f"per-call weights rank {r}")
    comb.run([z_arena] + [None] * (R - 1), y)
    torch.cuda.synchronize()
    want = OM.combine(z, idx, w, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want[r], f"routed weights again rank {r}")


def test_device_plan_unrouted_is_in_bounds():
    """Before the first route every slot is arena row 0: a copy is harmless."""
    require_gpu()
    T, h, E, k, R = 32, 8, 8, 2, 2
    disp = api.MoeDevicePlan(R, T, h, E, k, "dispatch")
    arena = empty_like_np(T * k * h, "bf16", 0)
    xs = [empty_like_np(T // R * h, "bf16", 3) for _ in range(R)]
    disp.run(xs, [arena] + [None] * (R - 1))
    torch.cuda.synchronize()
    a = from_dev(arena).reshape(T * k, h)
    assert np.all(a[1:] == 0) and np.all(a[0] == 3)


def test_device_routing_many_blocks():
    """262,144 tokens = 1024 routing blocks, more than can be resident at
    once: the three-kernel routing path (smaller token counts take the fused
    kernel).  Dispatch arena, rank offsets and combine against the oracle."""
    require_gpu()
    T, h, E, k, R = 262144, 8, 64, 2, 8
    rng = np.random.default_rng(91)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _run(T, h, E, k, R, idx, w, shards)


def _distinct_topk(rng, T, E, k, p=None):
    """T rows of k distinct experts, each drawn from p (uniform if None):
    rows with a repeat are drawn again until none is left."""
    idx = rng.choice(E, size=(T, k), p=p).astype(np.int32)
    while True:
        s = np.sort(idx, axis=1)
        bad = np.any(s[:, 1:] == s[:, :-1], axis=1)
        if not bad.any():
            return idx
        idx[bad] = rng.choice(E, size=(int(bad.sum()), k), p=p)


def test_device_routing_many_blocks_ragged_skewed():
    """The three-kernel routing path at the full workload's expert count and
    top-k: 266,664 tokens = 1041 full routing blocks and a ragged one of 168
    tokens, 256 experts over 8 ranks, top-8, expert choice skewed (weights
    1/(i+1)); dispatch arena, rank offsets and combine against the oracle."""
    require_gpu()
    T, h, E, k, R = 266664, 8, 256, 8, 8
    _say(f"device routing three-kernel: T={T} h={h} E={E} k={k} R={R} skewed")
    rng = np.random.default_rng(93)
    p = 1.0 / (np.arange(E) + 1.0)
    idx = _distinct_topk(rng, T, E, k, p / p.sum())
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _run(T, h, E, k, R, idx, w, shards)


def test_device_routing_many_blocks_max_experts():
    """The three-kernel routing path at the largest expert count and top-k
    the device routing takes (1024 experts, top-16; 262,144 tokens = 1024
    blocks): dispatch arena and rank offsets against the oracle.  The weight
    map goes through the same store as in the top-8 combine test."""
    require_gpu()
    T, h, E, k, R = 262144, 2, 1024, 16, 8
    _say(f"device routing three-kernel: T={T} h={h} E={E} k={k} R={R}")
    rng = np.random.default_rng(94)
    idx = _distinct_topk(rng, T, E, k)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    disp = api.MoeDevicePlan(R, T, h, E, k, "dispatch")
    offs = torch.zeros(R + 1, dtype=torch.int32, device=DEV)
    disp.route(torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV), offs)
    arena = empty_like_np(T * k * h, "bf16", -21555)
    disp.run([to_dev(s.reshape(-1)) for s in shards], [arena] + [None] * (R - 1))
    disp.check()
    _, counts, offsets, rows = OM.layout(idx, E, R)
    assert np.array_equal(offs.cpu().numpy(), np.concatenate([[0], np.cumsum(rows)]).astype(np.int32))
    want = np.concatenate(OM.dispatch(shards, idx, E), axis=0)
    assert_bits_equal(from_dev(arena).reshape(T * k, h), want, "three-kernel dispatch arena, 1024 experts")


@pytest.mark.parametrize("seed", range(4))
def test_device_routing_many_blocks_random(seed):
    """Seeded random shapes past the fused routing kernel's co-residency
    limit (80,000-100,000 tokens, 313-391 blocks with a ragged last one):
    the three-kernel path at random expert counts, top-k, rank counts,
    hidden sizes and skew; dispatch arena, rank offsets and combine
    against the oracle."""
    require_gpu()
    rng = np.random.default_rng([9005, seed])
    R = int(rng.choice([2, 4, 8]))
    T = R * (int(rng.integers(80000, 100001)) // R)
    E = min(1024, R * int(rng.choice([1, 4, 16, 64])))
    k = int(rng.choice([k for k in (1, 2, 3, 5, 8) if k <= E]))
    h = int(rng.choice([1, 3, 8]))
    p = None
    if rng.integers(0, 2):
        p = 1.0 / (np.arange(E) + 1.0)
        p = p / p.sum()
    _say(f"device routing three-kernel random {seed}: T={T} h={h} E={E} k={k} R={R} skew={p is not None}")
    idx = _distinct_topk(rng, T, E, k, p)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _run(T, h, E, k, R, idx, w, shards)


@pytest.mark.parametrize("seed", range(32))
def test_device_routing_random_shapes(seed):
    """Seeded random token counts (one to many blocks of 256, so the fused
    kernel and the three-kernel path both run), expert counts, top-k, rank
    counts and hidden sizes; expert choice uniform or skewed."""
    require_gpu()
    rng = np.random.default_rng([9004, seed])
    R = int(rng.choice([1, 2, 4, 8]))
    T = R * int(rng.choice([1, 3, 32, 100, 600, 4096]))
    E = R * int(rng.choice([1, 2, 8, 32]))
    k = int(rng.choice([k for k in (1, 2, 3, 4, 8, 16) if k <= E]))
    h = int(rng.choice([1, 8, 24, 64]))
    skew = bool(rng.integers(0, 2))
    _say(f"device routing random {seed}: T={T} h={h} E={E} k={k} R={R} skew={skew}")
    p = None
    if skew:
        p = 1.0 / (np.arange(E) + 1.0) ** 1.5
        p = p / p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _run(T, h, E, k, R, idx, w, shards)
