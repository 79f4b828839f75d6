"""GPU parity of SNAC chains of every layout-named collective (not only the
All-Reduce), through the C ABI: stage / notify / consume over a plan's index
map, for the barrier, dual-buffer, speculative and graph variants.  Every
epoch of every rank's output must equal the oracle's collective of that
epoch's inputs bit for bit, and outputs the plan does not write must keep
their sentinel.  Protocol stress as for the All-Reduce chain: staggered ranks
force mis-speculation, and a host-forced tiny poll budget must end in
RRB_ETIMEOUT rather than a hang."""

import sys

import numpy as np
import pytest
import torch

from oracle import chain as OC, collectives as C
from reduce_rank_buffers_amd import api, inputs
from reduce_rank_buffers_amd import _lib as L
from tests.gpu_util import DEV, assert_bits_equal, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = ["barrier", "dual", "speculative", "graph"]
LAYOUTS = {
    "all_reduce": (api.PARTIAL, api.REPLICATED, "reduce"),
    "reduce_scatter": (api.PARTIAL, api.SHARD, "reduce"),
    "all_gather": (api.SHARD, api.REPLICATED, "copy"),
    "all_to_all": (api.BLOCK_ROW, api.BLOCK_COL, "copy"),
    "broadcast": None,
    "reduce": None,
    "gather": None,
}
SHARD_INPUT = ("all_gather", "gather")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _layout(name, root):
    if name == "broadcast":
        return api.ROOT(root), api.REPLICATED, "copy"
    if name == "reduce":
        return api.PARTIAL, api.ROOT(root), "reduce"
    if name == "gather":
        return api.SHARD, api.ROOT(root), "copy"
    return LAYOUTS[name]


def _run_chain(name, R, n, dtype, variant, E=12, root=None, stagger=None, kind=0, slices=0):
    root = {"broadcast": 3, "reduce": 0, "gather": 5}.get(name, 0) % R if root is None else root
    lin, lout, op = _layout(name, root)
    plan = api.Plan(R, n, dtype, lin, lout, op)
    ch = api.SnacPlanChain(plan, variant, slices=slices)
    si, so = ch.strides
    per_rank_in = n // R if name in SHARD_INPUT else n
    if dtype == "bf16":
        ins = inputs.chain(E, R, per_rank_in, kind=200 + kind)
    else:
        rng = np.random.default_rng(300 + kind)
        ins = rng.standard_normal((E, R, per_rank_in)).astype(np.float32)
    host_in = np.zeros((E, R, si), dtype=ins.dtype)
    host_in[:, :, :per_rank_in] = ins
    inp = to_dev(host_in)
    out = torch.full((E, R, so), -21555 if dtype == "bf16" else -12345.0,
                     dtype=torch.int16 if dtype == "bf16" else torch.float32, device=DEV)
    stats = torch.zeros(4, dtype=torch.int64, device=DEV)
    ch.run(inp, out, stats=stats, stagger=stagger)
    ch.check()
    want = OC.collective_chain(name, [list(ins[e]) for e in range(E)], dtype, root=root)
    got = from_dev(out)
    sent = np.uint16(0xABCD) if dtype == "bf16" else np.float32(-12345.0)
    for e in range(E):
        for q in range(R):
            w = want[e][q]
            if w is None:
                assert np.all(got[e, q] == sent), f"{name} {variant} e={e}: rank {q} written"
            else:
                assert_bits_equal(got[e, q, :len(w)], w, f"{name} {variant} R={R} e={e} rank {q}")
    return stats.cpu().tolist(), ch


@pytest.mark.parametrize("name", list(LAYOUTS))
@pytest.mark.parametrize("variant", VARIANTS)
def test_plan_chain_bit_exact(name, variant):
    require_gpu()
    _say(f"plan chain {name} {variant}")
    st, ch = _run_chain(name, 8, 8 * 1024, "bf16", variant, kind=list(LAYOUTS).index(name))
    if variant != "graph":
        assert st[2] == 0 and st[3] == 12 * 8 * ch_slices(ch)


def ch_slices(ch):
    # epochs counted per (rank, slice) workgroup: recover the slice count
    return ch._slices if hasattr(ch, "_slices") else _default_slices(ch)


def _default_slices(ch):
    si, so = ch.strides
    nvec = max(si, so) * ch.esize // 16
    S = max(1, min(128, nvec // 64))
    return min(S, 2048 // ch.nranks, nvec)


@pytest.mark.parametrize("name", ["all_reduce", "reduce_scatter", "all_gather", "all_to_all"])
@pytest.mark.parametrize("R,n,dtype,slices", [(3, 3 * 256, "bf16", 0), (16, 16 * 512, "bf16", 0),
                                              (8, 8 * 2048, "f32", 0), (8, 8 * 4096, "bf16", 5),
                                              (2, 2 * 8, "bf16", 0)])
def test_plan_chain_other_shapes(name, R, n, dtype, slices):
    require_gpu()
    _say(f"plan chain {name} R={R} n={n} {dtype} slices={slices}")
    for variant in ("barrier", "dual", "speculative"):
        _run_chain(name, R, n, dtype, variant, E=6, kind=7, slices=slices)


@pytest.mark.parametrize("name", ["all_reduce", "reduce_scatter", "all_gather", "all_to_all",
                                  "broadcast", "reduce", "gather"])
def test_plan_chain_staggered_speculation(name):
    """Late ranks: the speculative consume sees stale flags, waits, reads the
    stale ranks' sources again, and every epoch is still exact (16 KiB per
    rank: every workgroup's work fits one round)."""
    require_gpu()
    R = 8
    st = [r * 64 for r in range(R)]
    stagger = torch.tensor(st, dtype=torch.int32, device=DEV)
    stats, _ = _run_chain(name, R, 8 * 1024, "bf16", "speculative", E=24, stagger=stagger, kind=9)
    _say(f"  {name}: misspec {stats[0]} retries {stats[1]}")
    assert stats[0] > 0
    # retries count the stale source ranks read after the wait that follows
    # a failed check (none when only write-after-read guards were stale)
    assert 0 <= stats[1] <= stats[0] * R
    for variant in ("barrier", "dual"):
        _run_chain(name, R, 8 * 1024, "bf16", variant, E=12, stagger=stagger, kind=9)


@pytest.mark.parametrize("name", ["all_reduce", "all_gather", "all_to_all", "reduce"])
@pytest.mark.parametrize("variant", ["barrier", "dual", "speculative"])
def test_plan_chain_stress_exact(name, variant):
    """4096 chained collectives over 32 seeded input sets (128 KiB tensor per
    rank, 64 workgroups per rank), every epoch of every rank bit-exact."""
    require_gpu()
    R, n, E, calls = 8, 8 * 8192, 32, 128
    root = {"reduce": 0}.get(name, 0)
    lin, lout, op = _layout(name, root)
    ch = api.SnacPlanChain(api.Plan(R, n, "bf16", lin, lout, op), variant)
    si, so = ch.strides
    per_rank_in = n // R if name in SHARD_INPUT else n
    ins = inputs.chain(E, R, per_rank_in, kind=260)
    host_in = np.zeros((E, R, si), dtype=ins.dtype)
    host_in[:, :, :per_rank_in] = ins
    inp = to_dev(host_in)
    want = OC.collective_chain(name, [list(ins[e]) for e in range(E)], "bf16", root=root)
    sent = np.uint16(0xABCD)
    want_np = np.full((E, R, so), sent, dtype=np.uint16)
    for e in range(E):
        for q in range(R):
            if want[e][q] is not None:
                want_np[e, q, :len(want[e][q])] = want[e][q]
    want_dev = to_dev(want_np)
    out = to_dev(np.full((E, R, so), sent, dtype=np.uint16))
    for c in range(calls):
        ch.run(inp, out)
        if not torch.equal(out, want_dev):
            ch.check()
            bad = (out != want_dev).nonzero()
            raise AssertionError(f"{name} {variant} mismatch in call {c} at {bad[:5].tolist()}")
    ch.check()


@pytest.mark.parametrize("name", ["all_gather", "all_to_all", "gather", "reduce_scatter"])
def test_plan_chain_large_staggered(name):
    """128 KiB tensors per rank (64 workgroups per rank, flat copy consume
    for the copies) with late ranks, every variant, every epoch bit-exact."""
    require_gpu()
    R = 8
    stagger = torch.tensor([r * 64 for r in range(R)], dtype=torch.int32, device=DEV)
    for variant in ("barrier", "dual", "speculative"):
        _run_chain(name, R, 8 * 8192, "bf16", variant, E=16, stagger=stagger, kind=11)


@pytest.mark.parametrize("name", ["all_reduce", "all_gather", "reduce_scatter"])
def test_plan_chain_two_part_speculation_staggered(name):
    """1 MiB tensors per rank: a workgroup's work takes several rounds, so
    the speculative consume runs the entries that read only current ranks,
    waits, then runs the rest; late ranks force that path, every epoch
    bit-exact."""
    require_gpu()
    R = 8
    stagger = torch.tensor([r * 64 for r in range(R)], dtype=torch.int32, device=DEV)
    stats, _ = _run_chain(name, R, 8 * 65536, "bf16", "speculative", E=6, stagger=stagger, kind=13)
    _say(f"  {name}: misspec {stats[0]} retries {stats[1]}")
    assert stats[0] > 0


def test_plan_chain_times_out_cleanly():
    require_gpu()
    R, n = 8, 8 * 1024
    plan = api.Plan(R, n, "bf16", api.SHARD, api.REPLICATED, "copy")
    st = [0] * R
    st[6] = 20000
    stagger = torch.tensor(st, dtype=torch.int32, device=DEV)
    for variant in ("barrier", "dual", "speculative"):
        ch = api.SnacPlanChain(plan, variant)
        si, so = ch.strides
        inp = torch.zeros((4, R, si), dtype=torch.int16, device=DEV)
        out = torch.empty((4, R, so), dtype=torch.int16, device=DEV)
        stats = torch.zeros(4, dtype=torch.int64, device=DEV)
        ch.run(inp, out, stats=stats, stagger=stagger, spin_limit=1)
        with pytest.raises(L.RrbError) as e:
            ch.check()
        assert e.value.status == L.RRB_ETIMEOUT
        assert stats.cpu().tolist()[2] > 0


def test_plan_chain_all_reduce_matches_all_reduce_chain():
    """The same All-Reduce chain through the plan-driven kernel and through
    the All-Reduce kernel gives the same bits."""
    require_gpu()
    R, n, E = 8, 4096, 8
    ins = inputs.chain(E, R, n, kind=77)
    inp = to_dev(ins)
    a = torch.empty_like(inp)
    b = torch.empty_like(inp)
    api.SnacChain(R, n, "bf16", "dual").run(inp, a)
    plan = api.Plan(R, n, "bf16", api.PARTIAL, api.REPLICATED, "reduce")
    pc = api.SnacPlanChain(plan, "dual")
    pc.run(inp, b)
    pc.check()
    assert torch.equal(a, b)


@pytest.mark.parametrize("variant", ["barrier", "dual", "speculative"])
def test_plan_chain_cooperative_launch(variant):
    require_gpu()
    R, n, E = 8, 8 * 1024, 8
    plan = api.Plan(R, n, "bf16", api.SHARD, api.REPLICATED, "copy")
    ch = api.SnacPlanChain(plan, variant, cooperative=True)
    si, so = ch.strides
    ins = inputs.chain(E, R, si, kind=250)
    inp = to_dev(ins)
    out = torch.empty((E, R, so), dtype=torch.int16, device=DEV)
    ch.run(inp, out)
    ch.check()
    want = OC.collective_chain("all_gather", [list(ins[e]) for e in range(E)])
    got = from_dev(out)
    for e in range(E):
        for q in range(R):
            assert_bits_equal(got[e, q], want[e][q], f"cooperative AG {variant} e={e} q={q}")
