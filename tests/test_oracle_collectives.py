"""Pins for the oracle's layout-named collectives (CPU only).

* brute force: per-element loops written straight from each collective's
  definition, against the closed forms;
* the generic naming definition (``oracle.collectives.collective``) against
  the closed forms for all seven, several R and n;
* invariants: all-gather after reduce-scatter equals all-reduce; all-to-all
  applied twice is the identity; all All-Reduce outputs are bit-identical;
  Reduce(root)[root] equals All-Reduce; Gather(root)[root] equals All-Gather;
  Broadcast outputs equal the root's input; non-root outputs are not written.
"""

import zlib

import numpy as np
import pytest

from oracle import bf16, collectives as C, fold
from tests import _exact


def _payloads(R, n, seed):
    rng = np.random.default_rng(seed)
    return [bf16.rne(rng.standard_normal(n).astype(np.float32)) for _ in range(R)]


def _brute(name, ins, R, n, root):
    c = n // R
    if name == "all_reduce":
        y = [_exact.fold_bf16_exact([int(x[j]) for x in ins]) for j in range(n)]
        return [np.array(y, dtype=np.uint16) for _ in range(R)]
    if name == "reduce_scatter":
        return [np.array([_exact.fold_bf16_exact([int(x[q * c + j]) for x in ins]) for j in range(c)],
                         dtype=np.uint16) for q in range(R)]
    if name == "reduce":
        out = [None] * R
        out[root] = np.array([_exact.fold_bf16_exact([int(x[j]) for x in ins]) for j in range(n)],
                             dtype=np.uint16)
        return out
    if name == "all_gather":
        outs = []
        for q in range(R):
            o = np.zeros(n, dtype=np.uint16)
            for r in range(R):
                for j in range(c):
                    o[r * c + j] = ins[r][j]
            outs.append(o)
        return outs
    if name == "gather":
        out = [None] * R
        o = np.zeros(n, dtype=np.uint16)
        for r in range(R):
            for j in range(c):
                o[r * c + j] = ins[r][j]
        out[root] = o
        return out
    if name == "broadcast":
        return [np.array([ins[root][j] for j in range(n)], dtype=np.uint16) for _ in range(R)]
    if name == "all_to_all":
        outs = []
        for q in range(R):
            o = np.zeros(n, dtype=np.uint16)
            for r in range(R):
                for j in range(c):
                    o[r * c + j] = ins[r][q * c + j]
            outs.append(o)
        return outs
    raise ValueError(name)


def _inputs_for(name, R, n, seed):
    c = n // R
    if name in ("all_gather", "gather"):
        return _payloads(R, c, seed)
    return _payloads(R, n, seed)


ROOTS = {"broadcast": 3, "reduce": 0, "gather": 5}


def _same(a, b):
    assert len(a) == len(b)
    for x, y in zip(a, b):
        if x is None or y is None:
            assert x is None and y is None
        else:
            assert np.array_equal(np.asarray(x), np.asarray(y))


@pytest.mark.parametrize("name", list(C.SEVEN))
@pytest.mark.parametrize("R,n", [(8, 16), (8, 64), (6, 24)])
def test_closed_form_vs_brute_force(name, R, n):
    root = ROOTS.get(name, 0) % R
    ins = _inputs_for(name, R, n, seed=zlib.crc32(f"{name}/{R}/{n}".encode()))
    got = C.named(name, ins, root=root)
    _same(got, _brute(name, ins, R, n, root))


@pytest.mark.parametrize("name", list(C.SEVEN))
@pytest.mark.parametrize("R,n", [(8, 64), (4, 32), (3, 12), (1, 8)])
def test_naming_definition_vs_closed_form(name, R, n):
    inl, outl, op = C.SEVEN[name]
    root = ROOTS.get(name, 0) % R
    if isinstance(inl, tuple):
        inl = C.ROOT(root)
    if isinstance(outl, tuple):
        outl = C.ROOT(root)
    ins = _inputs_for(name, R, n, seed=3)
    if name == "broadcast":
        ins = [x if r == root else None for r, x in enumerate(ins)]
    got = C.collective(inl, outl, op, ins, R, n)
    want = C.named(name, [x if x is not None else np.zeros(n, np.uint16) for x in ins], root=root)
    _same(got, want)


def test_invariants_R8():
    R, n = 8, 8 * 1000
    ins = _payloads(R, n, 11)
    ar = C.all_reduce(ins)
    for o in ar[1:]:
        assert np.array_equal(o, ar[0])
    rs = C.reduce_scatter(ins)
    ag = C.all_gather(rs)
    _same(ag, ar)
    a2a = C.all_to_all(ins)
    _same(C.all_to_all(a2a), ins)
    red = C.reduce_root(ins, 0)
    assert np.array_equal(red[0], ar[0]) and all(o is None for o in red[1:])
    shards = [x[: n // R] for x in ins]
    g = C.gather(shards, 5)
    assert np.array_equal(g[5], C.all_gather(shards)[0])
    assert sum(o is None for o in g) == R - 1
    b = C.broadcast(ins, 3)
    for o in b:
        assert np.array_equal(o, ins[3])


def test_f32_all_reduce_invariant():
    rng = np.random.default_rng(12)
    R, n = 8, 4096
    ins = [rng.standard_normal(n).astype(np.float32) for _ in range(R)]
    ar = C.all_reduce(ins, "f32")
    ag = C.all_gather(C.reduce_scatter(ins, "f32"))
    _same(ag, ar)
    assert ar[0].dtype == np.float32


def test_other_namings_scatter_and_slices():
    # Layout naming gives collectives beyond the seven: Scatter(root) is
    # ROOT -> SHARD copy; REPLICATED -> SHARD is a local slice.
    R, n = 4, 16
    ins = _payloads(R, n, 13)
    sc = C.collective(C.ROOT(2), C.SHARD, "copy", [None, None, ins[2], None], R, n)
    for q in range(R):
        assert np.array_equal(sc[q], ins[2][q * 4:(q + 1) * 4])
    sl = C.collective(C.REPLICATED, C.SHARD, "copy", ins, R, n)
    for q in range(R):
        assert np.array_equal(sl[q], ins[0][q * 4:(q + 1) * 4])


def test_invalid_specs_rejected():
    R, n = 4, 16
    ins = _payloads(R, n, 14)
    with pytest.raises(ValueError):
        C.collective(C.SHARD, C.REPLICATED, "reduce", ins, R, n)
    with pytest.raises(ValueError):
        C.collective(C.SHARD, C.BLOCK_COL, "copy", ins, R, n)
    with pytest.raises(ValueError):
        C.collective(C.SHARD, C.SHARD, "copy", ins, R, 18)


def test_ragged_all_reduce_any_n():
    R, n = 8, 37
    ins = _payloads(R, n, 15)
    got = C.collective(C.PARTIAL, C.REPLICATED, "reduce", ins, R, n)
    _same(got, C.all_reduce(ins))


def test_collective_chain_is_per_epoch_collective():
    """The chain oracle adds no orchestration: an All-Reduce chain equals the
    All-Reduce chain oracle on every rank, and an All-Gather chain's epoch e
    is the concatenation of that epoch's shards."""
    from oracle import chain as OC
    rng = np.random.default_rng(21)
    E, R, c = 3, 4, 8
    ins = [[bf16.rne(rng.standard_normal(R * c).astype(np.float32)) for _ in range(R)]
           for _ in range(E)]
    ar = OC.collective_chain("all_reduce", ins)
    for e, want in enumerate(OC.allreduce_chain(ins)):
        for q in range(R):
            assert np.array_equal(ar[e][q], want)
    shards = [[x[:c] for x in ins[e]] for e in range(E)]
    ag = OC.collective_chain("all_gather", shards)
    for e in range(E):
        for q in range(R):
            assert np.array_equal(ag[e][q], np.concatenate(shards[e]))
    g = OC.collective_chain("gather", shards, root=2)
    assert all(g[e][q] is None for e in range(E) for q in range(R) if q != 2)


@pytest.mark.parametrize("R", [3, 8])
def test_root_collectives_at_every_root(R):
    """Reduce, Gather and Broadcast at each root: the closed forms equal the
    element-by-element layout definition, the root gets the All-Reduce /
    All-Gather / its own buffer, and no other rank is written."""
    c = 4
    n = R * c
    ins = _payloads(R, n, 31 + R)
    shards = [x[:c] for x in ins]
    ar = C.all_reduce(ins)[0]
    ag = C.all_gather(shards)[0]
    for root in range(R):
        red = C.reduce_root(ins, root)
        _same(red, C.collective(C.PARTIAL, C.ROOT(root), "reduce", ins, R, n))
        assert np.array_equal(red[root], ar)
        assert all(red[q] is None for q in range(R) if q != root)
        gat = C.gather(shards, root)
        _same(gat, C.collective(C.SHARD, C.ROOT(root), "copy", shards, R, n))
        assert np.array_equal(gat[root], ag)
        assert all(gat[q] is None for q in range(R) if q != root)
        bc = C.broadcast(ins, root)
        _same(bc, C.collective(C.ROOT(root), C.REPLICATED, "copy",
                               [ins[q] if q == root else None for q in range(R)], R, n))
        assert all(np.array_equal(b, ins[root]) for b in bc)


def test_allreduce_chain_folds_in_fixed_rank_order():
    """Per epoch, every element of the chain oracle equals the exact rational
    emulation of the fixed-order fold, on data where the tree order differs:
    [2^24, 1, 1, -2^24] folds to 0 in rank order and to 1 pairwise."""
    from oracle import chain as OC
    from tests import _exact
    R, n, E = 4, 6, 3
    rng = np.random.default_rng(41)
    ins = []
    for e in range(E):
        xs = [bf16.rne((rng.standard_normal(n) * 2.0 ** rng.integers(-24, 25, n)).astype(np.float32))
              for _ in range(R)]
        for r, v in enumerate([2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)]):
            xs[r][0] = bf16.rne(np.array([v], dtype=np.float32))[0]
        ins.append(xs)
    got = OC.allreduce_chain(ins)
    for e in range(E):
        assert int(got[e][0]) == 0x0000
        for j in range(n):
            assert int(got[e][j]) == _exact.fold_bf16_exact([int(ins[e][r][j]) for r in range(R)])
