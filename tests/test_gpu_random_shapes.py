"""Seeded random-shape GPU parity: the seven layout-named collectives and
their SNAC plan chains over random rank counts, sizes, element types and
buffer alignments, each compared bit for bit with the oracle, with
sentinels on outputs a collective does not write.  The shapes mix tiny,
ragged (element path), one-workgroup, multi-tile and cache-sized blocks, so
every launch shape the library picks from a plan is reached without being
named."""

import sys

import numpy as np
import pytest
import torch

from oracle import chain as OC, collectives as C
from reduce_rank_buffers_amd import api
from tests.gpu_util import assert_bits_equal, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

ROOTED = ("broadcast", "reduce", "gather")
SHARD_INPUT = ("all_gather", "gather")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _payload(rng, m, dtype):
    x = rng.standard_normal(m).astype(np.float32) * np.float32(rng.choice([0.02, 1.0, 300.0]))
    if dtype == "f32":
        return x
    from oracle import bf16
    return bf16.rne(x)


def _dev_view(a, shift):
    """`a` on the device, starting `shift` elements into a larger buffer (so
    the view can be misaligned); the base is returned to keep it alive."""
    base = to_dev(np.concatenate([np.zeros(shift, a.dtype), a]))
    return base[shift:], base


def _case(seed):
    rng = np.random.default_rng([9001, seed])
    name = str(rng.choice(list(C.SEVEN)))
    R = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 11, 16]))
    dtype = str(rng.choice(["bf16", "f32"]))
    kind = rng.integers(0, 5)
    if kind == 0:
        c = int(rng.integers(1, 40))             # tiny
    elif kind == 1:
        c = 8 * int(rng.integers(1, 600))        # vector path, a few tiles
    elif kind == 2:
        c = 8 * int(rng.integers(600, 9000)) + int(rng.integers(0, 8))  # many tiles, maybe ragged
    elif kind == 3:
        c = int(rng.integers(1, 5000))           # anything
    else:
        c = 8 * 1024 * int(rng.integers(1, 9))   # around the small / split limits
    shift = int(rng.choice([0, 0, 0, 1, 3]))
    root = int(rng.integers(0, R))
    return rng, name, R, dtype, c, shift, root


@pytest.mark.parametrize("seed", range(320))
def test_random_collective(seed):
    require_gpu()
    rng, name, R, dtype, c, shift, root = _case(seed)
    n = R * c
    m = c if name in SHARD_INPUT else n
    _say(f"random {seed}: {name} R={R} c={c} {dtype} shift={shift} root={root}")
    ins_np = [_payload(rng, m, dtype) for _ in range(R)]
    want = C.named(name, ins_np, dtype, root=root if name in ROOTED else None)
    keep = []
    ins = []
    for x in ins_np:
        v, b = _dev_view(x, shift)
        ins.append(v)
        keep.append(b)
    sent = np.uint16(0xABCD) if dtype == "bf16" else np.float32(-12345.0)
    outs = []
    for w in want:
        length = n if w is None else len(w)
        v, b = _dev_view(np.full(length, sent), shift)
        outs.append(v)
        keep.append(b)
    fn = getattr(api, name)
    if name in ROOTED:
        fn(ins, outs, root)
    else:
        fn(ins, outs)
    torch.cuda.synchronize()
    for q, (o, w) in enumerate(zip(outs, want)):
        g = from_dev(o)
        if w is None:
            assert np.all(g == sent), f"{name} seed {seed}: rank {q} output was written"
        else:
            assert_bits_equal(g, w, f"{name} seed {seed} rank {q}")


LAYOUT = {
    "all_reduce": lambda r: (api.PARTIAL, api.REPLICATED, "reduce"),
    "reduce_scatter": lambda r: (api.PARTIAL, api.SHARD, "reduce"),
    "all_gather": lambda r: (api.SHARD, api.REPLICATED, "copy"),
    "all_to_all": lambda r: (api.BLOCK_ROW, api.BLOCK_COL, "copy"),
    "broadcast": lambda r: (api.ROOT(r), api.REPLICATED, "copy"),
    "reduce": lambda r: (api.PARTIAL, api.ROOT(r), "reduce"),
    "gather": lambda r: (api.SHARD, api.ROOT(r), "copy"),
}


@pytest.mark.parametrize("seed", range(96))
def test_random_plan_chain(seed):
    """SNAC chains of a random collective, variant, rank count, size and
    slice count (every map entry on 16-byte boundaries, as chains need)."""
    require_gpu()
    rng = np.random.default_rng([9002, seed])
    name = str(rng.choice(list(LAYOUT)))
    variant = str(rng.choice(["barrier", "dual", "speculative"]))
    R = int(rng.choice([2, 3, 4, 8, 16]))
    dtype = str(rng.choice(["bf16", "f32"]))
    per16 = 8 if dtype == "bf16" else 4
    c = per16 * int(rng.choice([1, 3, 16, 64, 200, 1024]))
    n = R * c
    root = int(rng.integers(0, R))
    slices = int(rng.choice([0, 0, 1, 3, 16]))
    E = 6
    _say(f"random chain {seed}: {name} {variant} R={R} c={c} {dtype} slices={slices} root={root}")
    lin, lout, op = LAYOUT[name](root)
    ch = api.SnacPlanChain(api.Plan(R, n, dtype, lin, lout, op), variant, slices=slices)
    si, so = ch.strides
    m = c if name in SHARD_INPUT else n
    ins = np.stack([np.stack([_payload(rng, m, dtype) for _ in range(R)]) for _ in range(E)])
    host_in = np.zeros((E, R, si), dtype=ins.dtype)
    host_in[:, :, :m] = ins
    sent = np.uint16(0xABCD) if dtype == "bf16" else np.float32(-12345.0)
    out = to_dev(np.full((E, R, so), sent))
    ch.run(to_dev(host_in), out)
    ch.check()
    want = OC.collective_chain(name, [list(ins[e]) for e in range(E)], dtype,
                               root=root if name in ROOTED else 0)
    got = from_dev(out)
    for e in range(E):
        for q in range(R):
            w = want[e][q]
            if w is None:
                assert np.all(got[e, q] == sent), f"{name} {variant} seed {seed}: rank {q} written"
            else:
                assert_bits_equal(got[e, q, :len(w)], w, f"{name} {variant} seed {seed} e={e} q={q}")


@pytest.mark.parametrize("seed", range(48))
def test_random_allreduce_chain(seed):
    """All-Reduce chains of a random variant, rank count, payload and slice
    count, every epoch of every rank bit-exact."""
    require_gpu()
    rng = np.random.default_rng([9005, seed])
    variant = str(rng.choice(["barrier", "dual", "speculative", "twoshot", "lamport", "graph"]))
    R = int(rng.choice([2, 3, 5, 8, 16]))
    dtype = "bf16" if variant == "lamport" else str(rng.choice(["bf16", "f32"]))
    per16 = 8 if dtype == "bf16" else 4
    n = per16 * int(rng.choice([1, 7, 64, 512, 1000, 8192]))
    slices = 0 if variant == "graph" else int(rng.choice([0, 0, 1, 5, 32]))
    E = 8
    _say(f"random all-reduce chain {seed}: {variant} R={R} n={n} {dtype} slices={slices}")
    ins = np.stack([np.stack([_payload(rng, n, dtype) for _ in range(R)]) for _ in range(E)])
    want = OC.allreduce_chain(ins, dtype)
    ch = api.SnacChain(R, n, dtype, variant, slices=slices)
    out = to_dev(np.zeros_like(ins))
    ch.run(to_dev(ins), out)
    ch.check()
    got = from_dev(out)
    for e in range(E):
        for r in range(R):
            assert_bits_equal(got[e, r], want[e], f"{variant} seed {seed} e={e} r={r}")
