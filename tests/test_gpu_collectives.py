"""GPU parity of the Atom copy / reduce kernels against the oracle, through the
C ABI.  Bit-exact: the fixed-order reduce and every copy have exactly one
correct bit pattern.  Workloads: the decode All-Reduce (8 x 4096 bf16), the
bandwidth sweep (1..256 MiB per rank, All-Reduce -> Reduce-Scatter ->
All-Gather, plus fp32 at 64 MiB), the seven layout-named collectives at 16 MiB
per rank, and edge cases (empty, ragged tails, unaligned layouts and
pointers, R from 1 to 16)."""

import sys

import numpy as np
import pytest
import torch

from oracle import collectives as C, fold
from reduce_rank_buffers_amd import api, inputs
from tests.gpu_util import (BF16_SPECIALS, DEV, assert_bits_equal, empty_like_np, from_dev,
                            oracle_elementwise, require_gpu, sentinel, to_dev)

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _run_and_check(name, ins_np, dtype, root=None):
    want = C.named(name, ins_np, dtype, root=root)
    ins = [to_dev(x) for x in ins_np]
    n_full = next(len(x) for x in want if x is not None)
    outs = [empty_like_np(n_full if w is None else len(w), dtype, sentinel(dtype)) for w in want]
    fn = getattr(api, name)
    if name in ("broadcast", "reduce", "gather"):
        fn(ins, outs, root)
    else:
        fn(ins, outs)
    torch.cuda.synchronize()
    for q, (o, w) in enumerate(zip(outs, want)):
        g = from_dev(o)
        if w is None:  # not written: still the sentinel
            assert np.all(g == (np.uint16(0xABCD) if dtype == "bf16" else np.float32(-12345.0))), \
                f"{name}: rank {q} output was written"
        else:
            assert_bits_equal(g, w, f"{name} rank {q}")


def test_decode_allreduce_bit_exact():
    require_gpu()
    ins = inputs.decode_allreduce()
    _say("decode all-reduce 8 x 4096 bf16")
    _run_and_check("all_reduce", ins, "bf16")


@pytest.mark.parametrize("S", [1, 4, 16])
def test_sweep_small_full_compare(S):
    require_gpu()
    _say(f"sweep S={S} MiB: AR, RS, AG full compare")
    ins = inputs.sweep(S)
    _run_and_check("all_reduce", ins, "bf16")
    _run_and_check("reduce_scatter", ins, "bf16")
    rs = C.reduce_scatter(ins)
    _run_and_check("all_gather", rs, "bf16")


def _full_sweep(S, dtype):
    """Full-size AR -> RS -> AG on the GPU, as the bench runs them (the
    streaming kernels with several vectors per lane run only at these sizes);
    every output element compared with the oracle's fixed-order fold."""
    R = 8
    ins_np = inputs.sweep(S, dtype=dtype)
    n = len(ins_np[0])
    c = n // R
    ins = [to_dev(x) for x in ins_np]
    ar = [empty_like_np(n, dtype) for _ in range(R)]
    rs = [empty_like_np(c, dtype) for _ in range(R)]
    ag = [empty_like_np(n, dtype) for _ in range(R)]
    api.all_reduce(ins, ar)
    api.reduce_scatter(ins, rs)
    api.all_gather(rs, ag)
    torch.cuda.synchronize()
    _say(f"  kernels: {api.bound('all_reduce', ins, ar).kernels()} | "
         f"{api.bound('reduce_scatter', ins, rs).kernels()} | {api.bound('all_gather', rs, ag).kernels()}")
    want = oracle_elementwise(lambda xs: fold.reduce(xs, dtype), ins_np)
    del ins
    for q in range(R):
        assert_bits_equal(from_dev(ar[q]), want, f"AR {S} MiB {dtype} rank {q}")
    for q in range(R):
        assert_bits_equal(from_dev(rs[q]), want[q * c:(q + 1) * c], f"RS {S} MiB {dtype} rank {q}")
    for q in range(R):
        assert_bits_equal(from_dev(ag[q]), want, f"AG(RS) {S} MiB {dtype} rank {q}")


@pytest.mark.parametrize("S", [64, 256])
def test_sweep_large_full_compare(S):
    require_gpu()
    _say(f"sweep S={S} MiB bf16, full compare")
    _full_sweep(S, "bf16")


def test_sweep_fp32_64mib_full_compare():
    require_gpu()
    _say("sweep fp32 64 MiB, full compare")
    _full_sweep(64, "f32")


ROOTS = {"broadcast": 3, "reduce": 0, "gather": 5}


@pytest.mark.parametrize("dtype,n", [("bf16", (1 << 24) + 5), ("f32", (1 << 23) + 3),
                                     ("bf16", (1 << 25) + 2)])
def test_unrolled_reduce_with_ragged_tail(dtype, n):
    """Single-segment reduces of 2M-4M vectors plus a ragged tail (four vectors
    per lane, then the element tail): All-Reduce and Reduce(root 2), full
    compare."""
    require_gpu()
    _say(f"unrolled reduce {dtype} n={n}")
    R = 8
    ins = inputs.rank_payloads(n, R, dtype, 1.0, inputs.WL_LARGE, 7)
    _run_and_check("all_reduce", ins, dtype)
    _run_and_check("reduce", ins, dtype, 2)


@pytest.mark.parametrize("name", list(C.SEVEN))
def test_seven_collectives_16mib(name):
    require_gpu()
    _say(f"seven: {name} 16 MiB")
    R = 8
    n = (16 << 20) // 2
    kind = list(C.SEVEN).index(name)
    if name in ("all_gather", "gather"):
        ins = inputs.rank_payloads(n // R, R, "bf16", 1.0, inputs.WL_SEVEN, kind)
    else:
        ins = inputs.rank_payloads(n, R, "bf16", 1.0, inputs.WL_SEVEN, kind)
    _run_and_check(name, ins, "bf16", ROOTS.get(name))


@pytest.mark.parametrize("name,R,c", [("gather", 8, 8 * 5001), ("all_to_all", 8, 8 * 5001),
                                      ("gather", 3, 8 * 9549), ("all_to_all", 5, 8 * 4097),
                                      ("gather", 1, 8 * 5001 + 3)])
def test_single_destination_copies_ragged(name, R, c):
    """Gather and All-to-All below the streaming size (two vectors per lane on
    128-lane workgroups) with blocks that are not a whole number of tiles, and
    one block with an element tail: full compare, sentinels outside the root."""
    require_gpu()
    _say(f"single-destination copy {name} R={R} c={c}")
    m = c if name == "gather" else R * c
    ins = inputs.rank_payloads(m, R, "bf16", 1.0, inputs.WL_SEVEN, 60 + R)
    _run_and_check(name, ins, "bf16", 5 % R if name == "gather" else None)


@pytest.mark.parametrize("R", [2, 3, 8, 16])
@pytest.mark.parametrize("c", [8, 8 * 64 + 8, 8 * 1024, 8 * 2048])
def test_small_fanout_all_gather(R, c):
    """All-Gathers of small shards (one workgroup per destination and tile up
    to 1024 vectors per shard, one per tile above): full compare."""
    require_gpu()
    _say(f"small fan-out all-gather R={R} c={c}")
    ins = inputs.rank_payloads(c, R, "bf16", 1.0, inputs.WL_SEVEN, 70 + R)
    _run_and_check("all_gather", ins, "bf16")


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 16])
@pytest.mark.parametrize("n", [0, 1, 7, 8, 37, 8 * 513 + 3, 4096])
def test_edge_all_reduce(R, n):
    require_gpu()
    rng = np.random.default_rng(R * 1000 + n)
    from oracle import bf16
    ins = [bf16.rne(rng.standard_normal(n).astype(np.float32)) for _ in range(R)]
    if n == 0:
        outs = [empty_like_np(0, "bf16") for _ in range(R)]
        api.all_reduce([to_dev(x) for x in ins], outs)
        torch.cuda.synchronize()
        return
    _run_and_check("all_reduce", ins, "bf16")


@pytest.mark.parametrize("name", list(C.SEVEN))
@pytest.mark.parametrize("R,c", [(8, 3), (8, 129), (3, 8), (16, 16), (4, 1)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_edge_block_layouts(name, R, c, dtype):
    """Block sizes not a multiple of 16 bytes take the element path."""
    require_gpu()
    root = ROOTS.get(name, 0) % R
    n = R * c
    rng = np.random.default_rng(R * 7 + c)
    from oracle import bf16
    gen = (lambda m: bf16.rne(rng.standard_normal(m).astype(np.float32))) if dtype == "bf16" \
        else (lambda m: rng.standard_normal(m).astype(np.float32))
    ins = [gen(c if name in ("all_gather", "gather") else n) for _ in range(R)]
    _run_and_check(name, ins, dtype, root if name in ROOTS else None)


def test_unaligned_pointers():
    """Views that start one element into an allocation are not 16-byte
    aligned; the library must still produce the exact result."""
    require_gpu()
    R, n = 8, 4096 + 5
    rng = np.random.default_rng(3)
    from oracle import bf16
    ins_np = [bf16.rne(rng.standard_normal(n).astype(np.float32)) for _ in range(R)]
    bases = [to_dev(np.concatenate([np.zeros(1, np.uint16), x])) for x in ins_np]
    ins = [b[1:] for b in bases]
    obases = [empty_like_np(n + 1, "bf16") for _ in range(R)]
    outs = [b[1:] for b in obases]
    api.all_reduce(ins, outs)
    torch.cuda.synchronize()
    want = C.all_reduce(ins_np)
    for q in range(R):
        assert_bits_equal(from_dev(outs[q]), want[q], f"unaligned AR rank {q}")


def test_special_values_and_denormals():
    require_gpu()
    R = 8
    vals = BF16_SPECIALS
    rng = np.random.default_rng(4)
    n = 8 * 4096
    ins = [vals[rng.integers(0, len(vals), size=n)] for _ in range(R)]
    _run_and_check("all_reduce", ins, "bf16")
    _run_and_check("reduce_scatter", ins, "bf16")


@pytest.mark.parametrize("R,n,dtype", [(3, (1 << 24) + 7, "bf16"), (5, (1 << 24) + 1, "bf16"),
                                       (5, (1 << 23) + 2, "f32"), (16, 1 << 20, "bf16"),
                                       (16, (1 << 20) + 5, "f32")])
def test_streaming_reduces_other_rank_counts(R, n, dtype):
    """Streaming launches at rank counts other than 8, full compare: the
    unrolled All-Reduce (non-temporal stores) and Reduce to a root
    (write-through stores) at 2M+ vectors with ragged tails, and at 16 ranks
    (one vector per lane) also the Reduce-Scatter."""
    require_gpu()
    _say(f"streaming reduces R={R} n={n} {dtype}")
    ins = inputs.rank_payloads(n, R, dtype, 1.0, inputs.WL_LARGE, 20 + R)
    _run_and_check("all_reduce", ins, dtype)
    _run_and_check("reduce", ins, dtype, R - 1)
    if n % R == 0:
        _run_and_check("reduce_scatter", ins, dtype)


@pytest.mark.parametrize("R", [4, 8])
@pytest.mark.parametrize("n", [37, 4096, 8 * 8192])
def test_fixed_rank_order_on_cancellation(R, n):
    """Elements whose rank-order fold differs from any other association
    ([2^24, 1, 1, -2^24, 0, ...] folds to 0 in rank order, to 1 pairwise)
    amid wide-range data: All-Reduce and Reduce-Scatter through the decode,
    vector and tail paths, against the oracle."""
    require_gpu()
    rng = np.random.default_rng(R * 10007 + n)
    from oracle import bf16
    ins = [bf16.rne((rng.standard_normal(n) * 2.0 ** rng.integers(-24, 25, n)).astype(np.float32))
           for _ in range(R)]
    col = bf16.rne(np.array([2.0 ** 24, 1.0, 1.0, -(2.0 ** 24)] + [0.0] * (R - 4), dtype=np.float32))
    for j in range(0, n, max(1, n // 64)):
        for r in range(R):
            ins[r][j] = col[r]
    assert C.all_reduce(ins)[0][0] == 0x0000
    _run_and_check("all_reduce", ins, "bf16")
    if n % R == 0:
        _run_and_check("reduce_scatter", ins, "bf16")


def test_invalid_call_arguments():
    """The library's own checks, called through the C ABI directly (the
    Python layer would reject these first): a NULL output of a rank the plan
    writes, a reduce entry point on a copy plan, weights on a layout-named
    reduce."""
    require_gpu()
    p = api.Plan(8, 64, "bf16", api.PARTIAL, api.REPLICATED, "reduce")
    from reduce_rank_buffers_amd import _lib as L
    ins = [empty_like_np(64, "bf16") for _ in range(8)]
    outs = [empty_like_np(64, "bf16") for _ in range(7)] + [None]
    st = L.lib().rrb_reduce(p.handle, api._ptrs(ins, 8), api._ptrs(outs, 8), None, api._stream())
    assert st == L.RRB_EINVAL
    with pytest.raises(ValueError):
        p.run(ins, outs)
    cp = api.Plan(8, 64, "bf16", api.SHARD, api.REPLICATED, "copy")
    with pytest.raises(L.RrbError):
        L.check(L.lib().rrb_reduce(cp.handle, api._ptrs(ins, 8), api._ptrs(ins, 8), None,
                                   api._stream()), "rrb_reduce")
    w = torch.ones(8, dtype=torch.float32, device=DEV)
    st = L.lib().rrb_reduce(p.handle, api._ptrs(ins, 8), api._ptrs(ins, 8), w.data_ptr(), api._stream())
    assert st == L.RRB_EINVAL


def test_graph_capture_replays_match_eager():
    """Atom launches captured in a HIP graph (torch.cuda.CUDAGraph over the
    library's stream argument) replay correctly several times, with eager
    input updates and synchronisations between replays."""
    require_gpu()
    R, n = 8, 4096
    sets = [inputs.rank_payloads(n, R, "bf16", 1.0, inputs.WL_DECODE, 10 + k) for k in range(3)]
    ins = [to_dev(x) for x in sets[0]]
    outs = [empty_like_np(n, "bf16") for _ in range(R)]
    rs = [empty_like_np(n // R, "bf16") for _ in range(R)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        api.all_reduce(ins, outs)
        api.reduce_scatter(ins, rs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.all_reduce(ins, outs)
        api.reduce_scatter(ins, rs)
    for k in range(3):
        for r in range(R):
            ins[r].copy_(to_dev(sets[k][r]))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = C.all_reduce(sets[k])
        want_rs = C.reduce_scatter(sets[k])
        for q in range(R):
            assert_bits_equal(from_dev(outs[q]), want[q], f"graph replay {k} AR rank {q}")
            assert_bits_equal(from_dev(rs[q]), want_rs[q], f"graph replay {k} RS rank {q}")


@pytest.mark.parametrize("name", list(C.SEVEN))
def test_bound_ops_match_oracle(name):
    """Pre-bound launches (plan and pointers resolved once) give the same bits,
    on repeated calls with new input contents."""
    require_gpu()
    R, n = 8, 8 * 1024
    root = ROOTS.get(name)
    m = n // R if name in ("all_gather", "gather") else n
    ins = [empty_like_np(m, "bf16") for _ in range(R)]
    want0 = C.named(name, [np.zeros(m, np.uint16)] * R, "bf16", root=root)
    n_full = next(len(x) for x in want0 if x is not None)
    outs = [empty_like_np(n_full if w is None else len(w), "bf16", sentinel("bf16")) for w in want0]
    op = api.bound(name, ins, outs, root=root)
    for k in range(2):
        host = inputs.rank_payloads(m, R, "bf16", 1.0, inputs.WL_SEVEN, 40 + k)
        for r in range(R):
            ins[r].copy_(to_dev(host[r]))
        op()
        torch.cuda.synchronize()
        for q, w in enumerate(C.named(name, host, "bf16", root=root)):
            if w is not None:
                assert_bits_equal(from_dev(outs[q]), w, f"bound {name} call {k} rank {q}")


def test_buffers_past_2_gib():
    """2.5 GiB per rank (byte offsets past 2^31): All-Reduce sampled against
    the oracle (including elements beyond the 2 GiB mark and the last ones),
    Reduce-Scatter sampled, and All-Gather of the Reduce-Scatter equal to the
    All-Reduce on all bytes."""
    require_gpu()
    R = 2
    n = ((5 << 30) // 2) // 2  # 2.5 GiB of bf16 per rank
    c = n // R
    _say(f"past 2 GiB: R={R} n={n}")
    ins = [inputs.device_normal_bf16(n, r, DEV, kind=1) for r in range(R)]
    ar = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(R)]
    api.all_reduce(ins, ar)
    rs = [torch.empty(c, dtype=torch.int16, device=DEV) for _ in range(R)]
    api.reduce_scatter(ins, rs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(61)
    edge = (1 << 31) // 2  # element at byte offset 2^31
    idx = np.unique(np.concatenate([rng.integers(0, n, size=1 << 16), np.arange(64),
                                    np.arange(n - 64, n), np.arange(edge - 32, edge + 32),
                                    np.arange(c - 8, c + 8)]))
    tidx = torch.from_numpy(idx).to(DEV)
    cols = [from_dev(x[tidx]) for x in ins]
    want = fold.reduce(cols, "bf16")
    for q in range(R):
        assert_bits_equal(from_dev(ar[q][tidx]), want, f"AR past 2 GiB rank {q}")
    for q in range(R):
        sel = (idx >= q * c) & (idx < (q + 1) * c)
        got = from_dev(rs[q][torch.from_numpy(idx[sel] - q * c).to(DEV)])
        assert_bits_equal(got, want[sel], f"RS past 2 GiB rank {q}")
    del ins
    ag = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(R)]
    api.all_gather(rs, ag)
    torch.cuda.synchronize()
    for q in range(R):
        assert torch.equal(ag[q], ar[0]), f"AG(RS) rank {q} differs from AR past 2 GiB"
        assert torch.equal(ar[q], ar[0])
