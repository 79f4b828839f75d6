"""GPU parity of the opt-in tree-order reduce (RRB_REDUCE_SUM_TREE) against
the oracle's tree-order fold, through the C ABI.  Bit-exact against that fold
(it has exactly one correct bit pattern); against the fixed-order fold it
must stay within max(1 bf16 ulp, 2 (R-1) 2^-24 sum |x|).  Inputs span
2^-24 .. 2^24 so that the fp32 partial sums round and the order matters."""

import sys

import numpy as np
import pytest
import torch

from oracle import collectives as C, fold
from reduce_rank_buffers_amd import api, inputs
from tests.gpu_util import (BF16_SPECIALS, DEV, assert_bits_equal, empty_like_np, from_dev,
                            oracle_elementwise, require_gpu, to_dev)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _wide(rng, n, dtype):
    x = rng.standard_normal(n, dtype=np.float32) * np.exp2(rng.integers(-24, 25, n).astype(np.float32))
    return inputs.to_bf16_bits(x) if dtype == "bf16" else x


@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 7, 8, 11, 16])
@pytest.mark.parametrize("n", [1, 7, 37, 4096, 8 * 513 + 3, 8 * 5000])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_tree_all_reduce_reduce_scatter_reduce(R, n, dtype):
    require_gpu()
    _say(f"tree R={R} n={n} {dtype}")
    rng = np.random.default_rng(R * 100003 + n)
    ins_np = [_wide(rng, n, dtype) for _ in range(R)]
    ins = [to_dev(x) for x in ins_np]
    want = fold.reduce_tree(ins_np, dtype)
    outs = [empty_like_np(n, dtype) for _ in range(R)]
    api.all_reduce(ins, outs, order="tree")
    if n % R == 0:
        c = n // R
        rs = [empty_like_np(c, dtype) for _ in range(R)]
        api.reduce_scatter(ins, rs, order="tree")
    root = R - 1
    red = [None] * R
    red[root] = empty_like_np(n, dtype)
    api.reduce(ins, red, root, order="tree")
    torch.cuda.synchronize()
    for q in range(R):
        assert_bits_equal(from_dev(outs[q]), want, f"tree AR rank {q}")
    if n % R == 0:
        for q in range(R):
            assert_bits_equal(from_dev(rs[q]), want[q * c:(q + 1) * c], f"tree RS rank {q}")
    assert_bits_equal(from_dev(red[root]), want, "tree Reduce root")


@pytest.mark.parametrize("R", [3, 8])
def test_tree_special_values(R):
    """Zeros, subnormals, infinities and NaNs of both signs with and without
    payload through the tree-order vector path (and its tail): every NaN
    result is 0x7FC0, the rest match the oracle's tree fold bit for bit."""
    require_gpu()
    rng = np.random.default_rng(11 + R)
    n = 8 * 4096 + 5
    ins_np = [BF16_SPECIALS[rng.integers(0, len(BF16_SPECIALS), size=n)] for _ in range(R)]
    want = fold.reduce_tree(ins_np, "bf16")
    outs = [empty_like_np(n, "bf16") for _ in range(R)]
    api.all_reduce([to_dev(x) for x in ins_np], outs, order="tree")
    torch.cuda.synchronize()
    for q in range(R):
        assert_bits_equal(from_dev(outs[q]), want, f"tree specials rank {q}")


def test_tree_collective_matches_layout_oracle():
    """The layout-named path with op reduce_tree, checked against the oracle's
    element-by-element collective."""
    require_gpu()
    R, n = 8, 8 * 300
    rng = np.random.default_rng(11)
    ins_np = [_wide(rng, n, "bf16") for _ in range(R)]
    want = C.collective(C.PARTIAL, C.SHARD, "reduce_tree", ins_np, R, n)
    outs = [empty_like_np(n // R, "bf16") for _ in range(R)]
    api.collective(api.PARTIAL, api.SHARD, "reduce_tree", [to_dev(x) for x in ins_np], outs, n)
    torch.cuda.synchronize()
    for q in range(R):
        assert_bits_equal(from_dev(outs[q]), want[q], f"tree RS (layout) rank {q}")


def test_tree_unaligned_pointers_take_element_path():
    require_gpu()
    R, n = 8, 4096 + 5
    rng = np.random.default_rng(12)
    ins_np = [_wide(rng, n, "bf16") for _ in range(R)]
    bases = [to_dev(np.concatenate([np.zeros(1, np.uint16), x])) for x in ins_np]
    obases = [empty_like_np(n + 1, "bf16") for _ in range(R)]
    api.all_reduce([b[1:] for b in bases], [b[1:] for b in obases], order="tree")
    torch.cuda.synchronize()
    want = fold.reduce_tree(ins_np, "bf16")
    for q in range(R):
        assert_bits_equal(from_dev(obases[q][1:]), want, f"unaligned tree AR rank {q}")


def test_tree_all_reduce_256mib_full_and_within_tolerance():
    """Full bench size and inputs (8 x 256 MiB bf16, N(0, 1)): every element
    of every replica bit-exact against the tree oracle; and, against the GPU's
    own fixed-order All-Reduce of the same data (itself pinned bit-exact by
    the collective tests), every element within the tolerance, checked on the
    device."""
    require_gpu()
    R = 8
    n = (256 << 20) // 2
    ins_np = inputs.sweep(256)  # the bench's own inputs
    ins = [to_dev(x) for x in ins_np]
    tree = [empty_like_np(n, "bf16") for _ in range(R)]
    fixed = [empty_like_np(n, "bf16") for _ in range(R)]
    api.all_reduce(ins, tree, order="tree")
    api.all_reduce(ins, fixed)
    torch.cuda.synchronize()
    want = oracle_elementwise(lambda xs: fold.reduce_tree(xs, "bf16"), ins_np)
    for q in range(R):
        assert_bits_equal(from_dev(tree[q]), want, f"tree AR 256 MiB rank {q}")

    def widen(t):
        return (t.to(torch.int32) << 16).view(torch.float32).to(torch.float64)
    ft, ff = widen(tree[0]), widen(fixed[0])
    mag = torch.zeros(n, dtype=torch.float64, device=DEV)
    for x in ins:
        mag += widen(x).abs()
    a = ff.abs().clamp_min(2.0 ** -126)
    ulp = torch.exp2(torch.floor(torch.log2(a)) - 7)
    tol = torch.maximum(ulp, 2 * (R - 1) * 2.0 ** -24 * mag)
    over = ((ft - ff).abs() > tol).sum().item()
    over_ulp = ((ft - ff).abs() > ulp).sum().item()
    differ = (tree[0] != fixed[0]).sum().item()
    _say(f"256 MiB: {differ} of {n} elements differ between orders; {over} beyond tolerance, "
         f"{over_ulp} beyond 1 bf16 ulp")
    assert over == 0
    assert over_ulp == 0  # on the workload's N(0, 1) data the plain 1-ulp rule holds


def test_tree_bound_op():
    """A pre-bound tree-order All-Reduce gives the tree oracle's bits."""
    require_gpu()
    R, n = 8, 8 * 1000
    rng = np.random.default_rng(14)
    ins_np = [_wide(rng, n, "bf16") for _ in range(R)]
    ins = [to_dev(x) for x in ins_np]
    outs = [empty_like_np(n, "bf16") for _ in range(R)]
    api.bound("all_reduce", ins, outs, order="tree")()
    torch.cuda.synchronize()
    want = fold.reduce_tree(ins_np, "bf16")
    for q in range(R):
        assert_bits_equal(from_dev(outs[q]), want, f"bound tree AR rank {q}")
