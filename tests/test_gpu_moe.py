"""GPU parity of MoE dispatch (row-map copy) and combine (weighted reduce in
ascending expert id) against the oracle, through the C ABI.  Full workload:
4096 tokens x 7168 bf16, 256 experts over 8 ranks, top-8 from the seeded gate;
plus small ragged shapes (hidden not a multiple of 8, other k)."""

import sys

import numpy as np
import pytest
import torch

from oracle import bf16, moe as OM
from reduce_rank_buffers_amd import api, inputs
from tests.gpu_util import BF16_SPECIALS, assert_bits_equal, empty_like_np, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _roundtrip(T, h, E, k, R, idx, w, x_shards, z_kind):
    disp = api.MoePlan(R, h, E, idx, w, "dispatch")
    comb = api.MoePlan(R, h, E, idx, w, "combine")
    xs = [to_dev(s.reshape(-1)) for s in x_shards]
    rows = disp.rows_per_rank
    recv = [empty_like_np(r * h, "bf16", -21555) for r in rows]
    disp.run(xs, recv)
    torch.cuda.synchronize()
    want_recv = OM.dispatch(x_shards, idx, E)
    for r in range(R):
        assert_bits_equal(from_dev(recv[r]).reshape(-1, h), want_recv[r], f"dispatch rank {r}")
    if z_kind == "identity":
        z_np = want_recv
        z = recv
    else:
        z_np = [bf16.rne(np.random.default_rng(50 + r).standard_normal((n, h)).astype(np.float32))
                for r, n in enumerate(rows)]
        z = [to_dev(a.reshape(-1)) for a in z_np]
    y = [empty_like_np(T // R * h, "bf16", -21555) for _ in range(R)]
    comb.run(z, y)
    torch.cuda.synchronize()
    want_y = OM.combine(z_np, idx, w, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want_y[r], f"combine rank {r}")


@pytest.mark.parametrize("z_kind", ["identity", "seeded"])
def test_moe_full_workload(z_kind):
    require_gpu()
    _say(f"moe full 4096 x 7168, z={z_kind}")
    T, h, E, k, R = 4096, 7168, 256, 8, 8
    idx, w = inputs.moe_routing(T, E, k)
    x = inputs.moe_tokens(T, h, R)
    _roundtrip(T, h, E, k, R, idx, w, x, z_kind)


@pytest.mark.parametrize("T,h,E,k,R", [(64, 24, 16, 4, 8), (32, 13, 8, 3, 4), (16, 8, 16, 16, 2),
                                       (8, 1, 4, 2, 2), (128, 7168, 32, 8, 8)])
def test_moe_shapes(T, h, E, k, R):
    require_gpu()
    rng = np.random.default_rng(T * h + k)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _roundtrip(T, h, E, k, R, idx, w, shards, "seeded")


def test_moe_skewed_routing():
    """Every token picks the same experts: one rank receives everything."""
    require_gpu()
    T, h, E, k, R = 256, 64, 32, 4, 8
    idx = np.tile(np.array([3, 1, 2, 0], dtype=np.int32), (T, 1))
    w = np.full((T, k), 0.25, dtype=np.float32)
    rng = np.random.default_rng(9)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _roundtrip(T, h, E, k, R, idx, w, shards, "identity")


# The fp32 weight whose exact product with 5.0 is 2^-8 + 2^-24 + 2^-33 (the
# oracle's MoE pins prove the premises): rounding the product before the add
# gives 1.0 (0x3F80) after 1.0 + product; a contracted multiply-add gives
# 0x3F81.
FMA_W_BITS = 978111898


def _combine_one_token(k, h, order, w_row, z_vals):
    """One token, R = 1, E = k: expert e's row is z_vals[e] in every column;
    the token's top-k list is `order` with weights `w_row`.  Returns the GPU
    combine row and the oracle's."""
    idx = np.array([order], dtype=np.int32)
    w = np.array([w_row], dtype=np.float32)
    z_np = [bf16.rne(np.repeat(np.array(z_vals, dtype=np.float32)[:, None], h, axis=1))]
    comb = api.MoePlan(1, h, k, idx, w, "combine")
    y = [empty_like_np(h, "bf16", -21555)]
    comb.run([to_dev(z_np[0].reshape(-1))], y)
    torch.cuda.synchronize()
    return from_dev(y[0]), OM.combine(z_np, idx, w, k, 1)[0].reshape(-1)


@pytest.mark.parametrize("k", [2, 4, 8])
@pytest.mark.parametrize("h", [8, 16, 13])
def test_combine_no_contraction_and_ascending_expert_order(k, h):
    """Crafted rows where a fused multiply-add, or folding in top-k order
    instead of ascending expert id, changes the bf16 result: the kernel
    (vector path for h = 8, 16; element path for h = 13) must match the
    oracle and the hand-derived bits."""
    require_gpu()
    w1 = float(np.array([FMA_W_BITS], dtype=np.uint32).view(np.float32)[0])
    # product rounding: experts 0 (z 1, w 1) and 1 (z 5, w w1), others 0
    z = [1.0, 5.0] + [0.0] * (k - 2)
    order = list(range(k))[::-1]
    w_row = [1.0 if e != 1 else w1 for e in order]
    got, want = _combine_one_token(k, h, order, w_row, z)
    assert np.all(want == 0x3F80)
    assert_bits_equal(got, want, f"combine rounding k={k} h={h}")
    if k >= 4:
        # order: 2^24 + 1 - 2^24 + 0... in ascending id is 0; the listed
        # top-k order 3, 1, 2, 0, ... would give 1
        z = [2.0 ** 24, 1.0, -(2.0 ** 24)] + [0.0] * (k - 3)
        order = [3, 1, 2, 0] + list(range(4, k))
        got, want = _combine_one_token(k, h, order, [1.0] * k, z)
        assert np.all(want == 0x0000)
        assert_bits_equal(got, want, f"combine order k={k} h={h}")


@pytest.mark.parametrize("h", [16, 13])
def test_combine_special_values(h):
    """Expert rows of zeros, subnormals, infinities and NaNs of both signs
    with and without payload through the vector (h = 16) and element
    (h = 13) combine paths: every NaN result is 0x7FC0, the rest match the
    oracle bit for bit."""
    require_gpu()
    T, E, k, R = 64, 16, 4, 8
    idx, w = inputs.moe_routing(T, E, k)
    comb = api.MoePlan(R, h, E, idx, w, "combine")
    rng = np.random.default_rng(7 + h)
    z_np = [BF16_SPECIALS[rng.integers(0, len(BF16_SPECIALS), size=(n, h))] for n in comb.rows_per_rank]
    y = [empty_like_np(T // R * h, "bf16", -21555) for _ in range(R)]
    comb.run([to_dev(a.reshape(-1)) for a in z_np], y)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore"):  # NaN and infinite inputs on purpose
        want = OM.combine(z_np, idx, w, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want[r], f"combine specials rank {r} h={h}")


@pytest.mark.parametrize("k", [17, 24, 32])
def test_moe_topk_above_16_vector_kernels(k):
    """Top-k above 16 (host-built maps only): the vector dispatch that reads
    slots per store and the vector combine that reads slots and weights per
    row, on full and ragged row parts; 64 experts over 8 ranks."""
    require_gpu()
    T, E, R = 64, 64, 8
    for h in (7168, 2392):
        rng = np.random.default_rng([9007, k, h])
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        w = rng.random((T, k)).astype(np.float32)
        xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
        shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
        _say(f"moe top-{k} h={h}")
        _roundtrip(T, h, E, k, R, idx, w, shards, "seeded")


@pytest.mark.parametrize("k", range(1, 17))
def test_moe_every_topk_vector_kernels(k):
    """Every top-k up to 16 has its own dispatch and combine kernels: full
    7168-wide rows (several row parts) and a 2392-wide row (299 vectors,
    a short last part), 64 tokens, 32 experts over 8 ranks."""
    require_gpu()
    T, E, R = 64, 32, 8
    for h in (7168, 2392):
        rng = np.random.default_rng([9006, k, h])
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        w = rng.random((T, k)).astype(np.float32)
        xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
        shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
        _say(f"moe top-{k} h={h}")
        _roundtrip(T, h, E, k, R, idx, w, shards, "seeded")


@pytest.mark.parametrize("seed", range(48))
def test_moe_random_shapes(seed):
    """Seeded random token counts, hidden sizes (vector and element paths, row
    parts with a short last part), expert counts, top-k (the vector kernels'
    k and others) and rank counts; expert choice uniform or skewed."""
    require_gpu()
    rng = np.random.default_rng([9003, seed])
    R = int(rng.choice([1, 2, 4, 8]))
    T = R * int(rng.integers(1, 65))
    E = R * int(rng.choice([1, 2, 4, 8, 32]))
    k = int(rng.choice([k for k in (1, 2, 3, 4, 6, 8, 16) if k <= E]))
    h = int(rng.choice([1, 7, 8, 24, 40, 8 * int(rng.integers(1, 300)), 7168]))
    skew = bool(rng.integers(0, 2))
    _say(f"moe random {seed}: T={T} h={h} E={E} k={k} R={R} skew={skew}")
    p = None
    if skew:
        p = 1.0 / (np.arange(E) + 1.0) ** 1.5
        p = p / p.sum()
    idx = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    xa = bf16.rne(rng.standard_normal((T, h)).astype(np.float32))
    shards = [xa[r * (T // R):(r + 1) * (T // R)] for r in range(R)]
    _roundtrip(T, h, E, k, R, idx, w, shards, str(rng.choice(["identity", "seeded"])))


@pytest.mark.parametrize("T,h,E,k,R", [(4096, 7168, 256, 8, 8), (64, 24, 16, 4, 8), (32, 13, 8, 3, 4),
                                       (16, 8, 16, 16, 2), (64, 2392, 64, 20, 8)])
def test_combine_per_call_weights(T, h, E, k, R):
    """rrb_reduce's d_weights on a host-built combine plan: weights given in
    the routing arrays' column order replace the plan's for one call (vector
    and element kernels); the next call without them uses the plan's again."""
    require_gpu()
    rng = np.random.default_rng(T * 31 + k)
    if T == 4096:
        idx, w = inputs.moe_routing(T, E, k)
    else:
        idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        w = rng.random((T, k)).astype(np.float32)
    w2 = (rng.standard_normal((T, k)) * 2).astype(np.float32)
    comb = api.MoePlan(R, h, E, idx, w, "combine")
    rows = [c // h for c in comb.in_count]
    z_np = [bf16.rne(rng.standard_normal((n, h)).astype(np.float32)) for n in rows]
    z = [to_dev(a.reshape(-1)) for a in z_np]
    y = [empty_like_np(T // R * h, "bf16", -21555) for _ in range(R)]
    comb.run(z, y, weights=torch.from_numpy(w2).to(z[0].device))
    torch.cuda.synchronize()
    want2 = OM.combine(z_np, idx, w2, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want2[r], f"per-call weights rank {r}")
    comb.run(z, y)
    torch.cuda.synchronize()
    want = OM.combine(z_np, idx, w, E, T // R)
    for r in range(R):
        assert_bits_equal(from_dev(y[r]).reshape(-1, h), want[r], f"plan weights rank {r}")
