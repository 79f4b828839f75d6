"""C ABI on the host (no GPU): the library loads, exports every symbol the
header declares, and its plan builder produces index maps that, applied to
buffers by a plain Python interpreter of rrb_segment, give exactly the
oracle's collectives."""

import os
import re

import numpy as np
import pytest

from oracle import collectives as C, fold, moe as OM
from reduce_rank_buffers_amd import _lib as L
from reduce_rank_buffers_amd import api

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "rrb.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rrb_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(librrb):
    names = _declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(librrb, n), n
    assert set(names) == set(L.EXPORTS)
    assert librrb.rrb_abi_version() == 2


def test_fenced_build_exports_reports_and_refuses_flag_in_data(librrb):
    """librrb_fenced.so (the chains' memory-model ordering) exports the same
    symbols, reports its ordering, and refuses only the flag-in-data chain,
    which has no fenced form; the default library reports no fences."""
    import ctypes
    fenced = L._open(L.LIB_FENCED_PATH)
    plain = L._open(L.LIB_PATH)
    for n in _declared():
        assert hasattr(fenced, n), n
    assert fenced.rrb_abi_version() == plain.rrb_abi_version()
    assert plain.rrb_snac_fenced() == 0 and fenced.rrb_snac_fenced() == 1
    lam = L.RRB_SNAC_LAMPORT | L.RRB_SNAC_DUAL_BUFFER
    h = ctypes.c_void_p()
    st = fenced.rrb_snac_create(8, 4096, 0, lam, 0, ctypes.byref(h))
    assert st == L.RRB_EUNSUPPORTED
    assert b"fenced" in fenced.rrb_last_error()
    # the message comes from the library the call went to, not lib()
    assert plain.rrb_snac_create(8, 4096, 0, 1 << 20, 0, ctypes.byref(h)) == L.RRB_EINVAL
    with pytest.raises(L.RrbError, match="fenced"):
        L.check(st, "rrb_snac_create", fenced)
    assert plain.rrb_snac_create(8, 4096, 0, lam, 0, ctypes.byref(h)) == L.RRB_OK
    plain.rrb_snac_destroy(h)
    for f in (0, L.RRB_SNAC_DUAL_BUFFER, L.RRB_SNAC_DUAL_BUFFER | L.RRB_SNAC_SPECULATIVE,
              L.RRB_SNAC_DUAL_BUFFER | L.RRB_SNAC_TWOSHOT, L.RRB_SNAC_GRAPH):
        h = ctypes.c_void_p()
        assert fenced.rrb_snac_create(8, 4096, 0, f, 0, ctypes.byref(h)) == L.RRB_OK, f
        fenced.rrb_snac_destroy(h)


def test_library_selection_switches_and_restores(librrb):
    prev = L.select(True)
    try:
        assert L.lib().rrb_snac_fenced() == 1
    finally:
        L.restore(prev)
    assert L.lib() is librrb


def _apply(segments, ins, in_count, out_count, R, dtype):
    """Interpret a plan's index map on numpy buffers (sentinel-filled outputs)."""
    dt = np.uint16 if dtype == "bf16" else np.float32
    sentinel = dt(0xABCD) if dtype == "bf16" else np.float32(-12345.0)
    outs = [np.full(int(c), sentinel, dtype=dt) for c in out_count]
    for src_rank, so, do, ln, mask in segments:
        if src_rank < 0:
            val = fold.reduce([ins[r][so:so + ln] for r in range(R)], dtype)
        else:
            val = ins[src_rank][so:so + ln]
        for q in range(R):
            if mask >> q & 1:
                outs[q][do:do + ln] = val
    return [o if c else None for o, c in zip(outs, out_count)]


def _payloads(R, n, dtype, seed):
    rng = np.random.default_rng(seed)
    if dtype == "f32":
        return [rng.standard_normal(n).astype(np.float32) for _ in range(R)]
    from oracle import bf16
    return [bf16.rne(rng.standard_normal(n).astype(np.float32)) for _ in range(R)]


ROOTS = {"broadcast": 3, "reduce": 0, "gather": 5}


@pytest.mark.parametrize("name", list(C.SEVEN))
@pytest.mark.parametrize("R,n", [(8, 64), (8, 8 * 37), (4, 32), (3, 12), (1, 8), (5, 40)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plan_map_equals_oracle(librrb, name, R, n, dtype):
    inl, outl, op = C.SEVEN[name]
    root = ROOTS.get(name, 0) % R
    kind = lambda l: api.ROOT(root) if isinstance(l, tuple) else getattr(api, l)
    p = api.Plan(R, n, dtype, kind(inl), kind(outl), op)
    segs = p.segments()
    c = n // R
    if name in ("all_gather", "gather"):
        ins = _payloads(R, c, dtype, 1)
    else:
        ins = _payloads(R, n, dtype, 1)
    got = _apply(segs, ins, p.in_count, p.out_count, R, dtype)
    want = C.named(name, ins, dtype, root=root)
    for g, w in zip(got, want):
        if w is None:
            assert g is None
        else:
            assert np.array_equal(g.view(np.uint8), np.asarray(w).view(np.uint8))
    # sizes the plan asks for match the layouts
    for r in range(R):
        assert p.in_count[r] == (0 if (name == "broadcast" and r != root) else len(ins[r]))


def test_fan_out_and_fusion_shapes(librrb):
    R, n = 8, 8 * 1024
    ar = api.Plan(R, n, "bf16", api.PARTIAL, api.REPLICATED, "reduce").segments()
    assert ar == [(-1, 0, 0, n, 0xFF)]  # one segment, read once, written 8 times
    rs = api.Plan(R, n, "bf16", api.PARTIAL, api.SHARD, "reduce").segments()
    assert sorted(rs) == sorted((-1, q * 1024, 0, 1024, 1 << q) for q in range(R))
    ag = api.Plan(R, n, "bf16", api.SHARD, api.REPLICATED, "copy").segments()
    assert sorted(ag) == sorted((r, 0, r * 1024, 1024, 0xFF) for r in range(R))
    a2a = api.Plan(R, n, "bf16", api.BLOCK_ROW, api.BLOCK_COL, "copy").segments()
    assert len(a2a) == 64
    bc = api.Plan(R, n, "bf16", api.ROOT(3), api.REPLICATED, "copy").segments()
    assert bc == [(3, 0, 0, n, 0xFF)]


def test_other_namings(librrb):
    R, n = 4, 32
    ins = _payloads(R, n, "bf16", 2)
    for inl, outl, op, ol in [
        (api.ROOT(2), api.SHARD, "copy", (C.ROOT(2), C.SHARD)),
        (api.REPLICATED, api.SHARD, "copy", (C.REPLICATED, C.SHARD)),
        (api.SHARD, api.SHARD, "copy", (C.SHARD, C.SHARD)),
        (api.REPLICATED, api.ROOT(1), "copy", (C.REPLICATED, C.ROOT(1))),
        (api.BLOCK_COL, api.BLOCK_ROW, "copy", (C.BLOCK_COL, C.BLOCK_ROW)),
    ]:
        p = api.Plan(R, n, "bf16", inl, outl, op)
        src = [x if p.in_count[r] else None for r, x in enumerate(ins)]
        src = [x[:p.in_count[r]] if x is not None else None for r, x in enumerate(src)]
        got = _apply(p.segments(), src, p.in_count, p.out_count, R, "bf16")
        want = C.collective(ol[0], ol[1], op, src, R, n)
        for g, w in zip(got, want):
            assert (g is None) == (w is None)
            if w is not None:
                assert np.array_equal(g, w)


@pytest.mark.parametrize("spec,msg", [
    ((8, 64, api.SHARD, api.REPLICATED, "reduce"), "PARTIAL input"),
    ((8, 64, api.PARTIAL, api.REPLICATED, "copy"), "reduce op"),
    ((8, 60, api.PARTIAL, api.SHARD, "reduce"), "count % nranks"),
    ((8, 64, api.SHARD, api.BLOCK_COL, "copy"), "only pair"),
    ((8, 64, api.PARTIAL, api.ROOT(9), "reduce"), "root"),
    ((17, 64, api.PARTIAL, api.REPLICATED, "reduce"), "nranks"),
    ((8, 64, api.REPLICATED, api.PARTIAL, "copy"), "cannot be an output"),
    ((8, 64, api.ROOT(1), api.BLOCK_COL, "copy"), "only pair"),
    ((8, 64, api.SHARD, api.REPLICATED, "reduce_tree"), "PARTIAL input"),
    ((8, 64, api.PARTIAL, api.REPLICATED, 3), "unknown op"),
])
def test_invalid_specs(librrb, spec, msg):
    R, n, i, o, op = spec
    with pytest.raises(L.RrbError) as e:
        api.Plan(R, n, "bf16", i, o, op)
    assert e.value.status == L.RRB_EINVAL
    assert msg in str(e.value)


def test_tree_op_plans_like_reduce(librrb):
    """The tree order changes only the fold inside the kernel: the index map
    is the fixed-order reduce's."""
    for out in (api.REPLICATED, api.SHARD, api.ROOT(2)):
        a = api.Plan(8, 64, "bf16", api.PARTIAL, out, "reduce")
        b = api.Plan(8, 64, "bf16", api.PARTIAL, out, "reduce_tree")
        assert a.segments() == b.segments()
        assert (a.in_count, a.out_count) == (b.in_count, b.out_count)
        assert b.op == L.RRB_REDUCE_SUM_TREE


def test_zero_count_plan(librrb):
    p = api.Plan(8, 0, "bf16", api.PARTIAL, api.REPLICATED, "reduce")
    assert p.in_count == [0] * 8 and p.out_count == [0] * 8


def test_segments_out_may_be_null_only_without_capacity(librrb):
    import ctypes
    lib = librrb
    p = api.Plan(8, 4096, "bf16", api.SHARD, api.REPLICATED, "copy")
    n = ctypes.c_int32(-1)
    L.check(lib.rrb_plan_segments(p.handle, None, 0, ctypes.byref(n)), "count only")
    assert n.value == len(p.segments()) > 0
    assert lib.rrb_plan_segments(p.handle, None, 4, ctypes.byref(n)) == L.RRB_EINVAL
    assert b"NULL out" in lib.rrb_last_error()


@pytest.mark.parametrize("T,E,k,R", [(64, 32, 4, 8), (4096, 256, 8, 8), (32, 8, 8, 4)])
def test_row_plan_sizes_match_oracle(librrb, T, E, k, R):
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k)).astype(np.float32)
    h = 16
    _, counts, offsets, rows = OM.layout(idx, E, R)
    import ctypes
    lib = L.lib()
    for d, name in ((L.RRB_MOE_DISPATCH, "dispatch"), (L.RRB_MOE_COMBINE, "combine")):
        hdl = ctypes.c_void_p()
        L.check(lib.rrb_plan_create_rows(R, T, h, E, k, idx.ctypes.data, w.ctypes.data, d,
                                         ctypes.byref(hdl)), "rows")
        ws = ctypes.c_size_t()
        inc = (ctypes.c_int64 * R)()
        outc = (ctypes.c_int64 * R)()
        L.check(lib.rrb_plan_query(hdl, ctypes.byref(ws), inc, outc), "query")
        recv = [int(x) * h for x in rows]
        tok = [T // R * h] * R
        if name == "dispatch":
            assert list(inc) == tok and list(outc) == recv
        else:
            assert list(inc) == recv and list(outc) == tok
        assert ws.value >= 2 * T * k * 4
        lib.rrb_plan_destroy(hdl)


def test_row_plans_reject_rows_of_2_gib(librrb):
    import ctypes
    lib = librrb
    h = 1 << 30  # 2 GiB of bf16 per row
    idx = np.zeros((8, 1), dtype=np.int32)
    hdl = ctypes.c_void_p()
    assert lib.rrb_plan_create_rows(8, 8, h, 8, 1, idx.ctypes.data, None, 0,
                                    ctypes.byref(hdl)) == L.RRB_EUNSUPPORTED
    assert b"2 GiB" in lib.rrb_last_error()
    assert lib.rrb_plan_create_rows_device(8, 8, h, 8, 1, 1, ctypes.byref(hdl)) == L.RRB_EUNSUPPORTED


def test_row_plan_rejects_bad_routing(librrb):
    import ctypes
    lib = L.lib()
    idx = np.array([[0, 0], [1, 2]], dtype=np.int32)
    w = np.ones((2, 2), dtype=np.float32)
    hdl = ctypes.c_void_p()
    st = lib.rrb_plan_create_rows(2, 2, 8, 4, 2, idx.ctypes.data, w.ctypes.data, 0, ctypes.byref(hdl))
    assert st == L.RRB_EINVAL and b"twice" in lib.rrb_last_error()
    idx = np.array([[0, 7], [1, 2]], dtype=np.int32)
    st = lib.rrb_plan_create_rows(2, 2, 8, 4, 2, idx.ctypes.data, w.ctypes.data, 0, ctypes.byref(hdl))
    assert st == L.RRB_EINVAL and b"expert 7" in lib.rrb_last_error()


def test_snac_create_validation(librrb):
    import ctypes
    lib = L.lib()
    h = ctypes.c_void_p()
    assert lib.rrb_snac_create(8, 4096, 0, 2, 0, ctypes.byref(h)) == L.RRB_EINVAL  # spec w/o dual
    assert lib.rrb_snac_create(8, 4095, 0, 1, 0, ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_snac_create(0, 4096, 0, 1, 0, ctypes.byref(h)) == L.RRB_EINVAL
    assert lib.rrb_snac_create(8, 4096, 0, 5, 0, ctypes.byref(h)) == L.RRB_EINVAL  # graph + dual
    assert lib.rrb_snac_create(8, 4096, 0, 8, 0, ctypes.byref(h)) == L.RRB_EINVAL  # twoshot alone
    assert lib.rrb_snac_create(8, 4096, 0, 11, 0, ctypes.byref(h)) == L.RRB_EINVAL  # + speculative
    assert lib.rrb_snac_create(8, 4096, 0, 9, 0, ctypes.byref(h)) == L.RRB_OK
    lib.rrb_snac_destroy(h)
    assert lib.rrb_snac_create(8, 4096, 0, 16, 0, ctypes.byref(h)) == L.RRB_EINVAL  # lamport alone
    assert lib.rrb_snac_create(8, 4096, 0, 19, 0, ctypes.byref(h)) == L.RRB_EINVAL  # + speculative
    assert lib.rrb_snac_create(8, 4096, 0, 25, 0, ctypes.byref(h)) == L.RRB_EINVAL  # + twoshot
    assert lib.rrb_snac_create(8, 4096, 0, L.RRB_SNAC_COOPERATIVE | L.RRB_SNAC_GRAPH, 0,
                               ctypes.byref(h)) == L.RRB_EINVAL
    assert lib.rrb_snac_create(8, 4096, 0, L.RRB_SNAC_COOPERATIVE | 1, 0, ctypes.byref(h)) == L.RRB_OK
    lib.rrb_snac_destroy(h)
    assert lib.rrb_snac_create(8, 4096, 0, L.RRB_SNAC_COOPERATIVE | 17, 0, ctypes.byref(h)) == L.RRB_OK
    lib.rrb_snac_destroy(h)
    assert lib.rrb_snac_create(8, 4096, 0, 17, 0, ctypes.byref(h)) == L.RRB_OK
    ws = ctypes.c_size_t()
    assert lib.rrb_snac_workspace(h, ctypes.byref(ws)) == L.RRB_OK
    # two tagged buffers of 8 ranks x 4096 bf16 halves, 4 bytes each, + status
    assert ws.value == 2 * 8 * 4096 * 4 + 256
    lib.rrb_snac_destroy(h)
    assert lib.rrb_snac_create(8, 4096, 0, 4, 0, ctypes.byref(h)) == L.RRB_OK
    lib.rrb_snac_destroy(h)
    # always-speculate goes with the speculative variant only
    for f in (L.RRB_SNAC_SPEC_ALWAYS, L.RRB_SNAC_SPEC_ALWAYS | 1, L.RRB_SNAC_SPEC_ALWAYS | 9,
              L.RRB_SNAC_SPEC_ALWAYS | 17, L.RRB_SNAC_SPEC_ALWAYS | 4):
        assert lib.rrb_snac_create(8, 4096, 0, f, 0, ctypes.byref(h)) == L.RRB_EINVAL, f
    assert lib.rrb_snac_create(8, 4096, 0, L.RRB_SNAC_SPEC_ALWAYS | 3, 0, ctypes.byref(h)) == L.RRB_OK
    lib.rrb_snac_destroy(h)
    assert lib.rrb_snac_create(8, 4096, 0, 128, 0, ctypes.byref(h)) == L.RRB_EINVAL  # unknown bit
    assert lib.rrb_snac_create(8, 4096, 0, 3, 0, ctypes.byref(h)) == L.RRB_OK
    ws = ctypes.c_size_t()
    assert lib.rrb_snac_workspace(h, ctypes.byref(ws)) == L.RRB_OK
    assert ws.value >= 2 * 8 * 4096 * 2
    # unbound handle refuses to run
    assert lib.rrb_snac_allreduce_chain(h, 1, None, None, None, None, 0, None) == L.RRB_EINVAL
    lib.rrb_snac_destroy(h)


def test_device_row_plan_sizes_and_limits(librrb):
    import ctypes
    lib = L.lib()
    R, T, h, E, k = 8, 4096, 7168, 256, 8
    for d in (L.RRB_MOE_DISPATCH, L.RRB_MOE_COMBINE):
        hdl = ctypes.c_void_p()
        L.check(lib.rrb_plan_create_rows_device(R, T, h, E, k, d, ctypes.byref(hdl)), "dev rows")
        ws = ctypes.c_size_t()
        inc = (ctypes.c_int64 * R)()
        outc = (ctypes.c_int64 * R)()
        L.check(lib.rrb_plan_query(hdl, ctypes.byref(ws), inc, outc), "query")
        arena = [T * k * h] + [0] * (R - 1)
        tok = [T // R * h] * R
        if d == L.RRB_MOE_DISPATCH:
            assert list(inc) == tok and list(outc) == arena
        else:
            assert list(inc) == arena and list(outc) == tok
        assert ws.value >= 2 * T * k * 4
        # routing before binding is refused
        assert lib.rrb_moe_route(hdl, None, None, None, None) == L.RRB_EINVAL
        lib.rrb_plan_destroy(hdl)
    hdl = ctypes.c_void_p()
    assert lib.rrb_plan_create_rows_device(R, T, h, 2048, k, 0, ctypes.byref(hdl)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_plan_create_rows_device(R, T, h, E, 17, 0, ctypes.byref(hdl)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_plan_create_rows_device(R, T + 1, h, E, k, 0, ctypes.byref(hdl)) == L.RRB_EINVAL


def test_snac_plan_chain_validation(librrb):
    """rrb_snac_create_plan: plans, flags and alignment it refuses; strides
    and workspace of one it accepts (host only, no kernel runs)."""
    import ctypes
    lib = L.lib()
    h = ctypes.c_void_p()
    ag = api.Plan(8, 8 * 64, "bf16", api.SHARD, api.REPLICATED, "copy")
    assert lib.rrb_snac_create_plan(ag.handle, L.RRB_SNAC_LAMPORT | L.RRB_SNAC_DUAL_BUFFER, 0,
                                    ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_snac_create_plan(ag.handle, L.RRB_SNAC_SPECULATIVE, 0,
                                    ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    tree = api.Plan(8, 8 * 64, "bf16", api.PARTIAL, api.REPLICATED, "reduce_tree")
    assert lib.rrb_snac_create_plan(tree.handle, 1, 0, ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    ragged = api.Plan(8, 8 * 3, "bf16", api.SHARD, api.REPLICATED, "copy")
    assert lib.rrb_snac_create_plan(ragged.handle, 1, 0, ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_snac_create_plan(None, 1, 0, ctypes.byref(h)) == L.RRB_EINVAL
    # plan chains speculate at every size; the All-Reduce chain's override is refused
    assert lib.rrb_snac_create_plan(ag.handle, L.RRB_SNAC_SPEC_ALWAYS | 3, 0,
                                    ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_snac_create_plan(ag.handle, L.RRB_SNAC_COOPERATIVE | L.RRB_SNAC_GRAPH, 0,
                                    ctypes.byref(h)) == L.RRB_EUNSUPPORTED
    assert lib.rrb_snac_create_plan(ag.handle, L.RRB_SNAC_COOPERATIVE | 1, 0,
                                    ctypes.byref(h)) == L.RRB_OK
    lib.rrb_snac_destroy(h)
    assert lib.rrb_snac_create_plan(ag.handle, 1, 0, ctypes.byref(h)) == L.RRB_OK
    si, so = ctypes.c_int64(), ctypes.c_int64()
    assert lib.rrb_snac_strides(h, ctypes.byref(si), ctypes.byref(so)) == L.RRB_OK
    assert (si.value, so.value) == (64 * 2, 8 * 64 * 2)
    ws = ctypes.c_size_t()
    assert lib.rrb_snac_workspace(h, ctypes.byref(ws)) == L.RRB_OK
    assert ws.value >= 2 * 8 * 128 + 256
    # a plan chain does not run through the All-Reduce entry point
    assert lib.rrb_snac_allreduce_chain(h, 1, None, None, None, None, 0, None) == L.RRB_EINVAL
    lib.rrb_snac_destroy(h)
    del ag  # the handle keeps its own copy of the plan


def test_missing_library_fails_loudly(tmp_path):
    """No fallback: with the shared library absent every entry point raises
    instead of computing anywhere else (checked in a fresh interpreter so
    this process's loaded library is untouched)."""
    import subprocess
    import sys as _sys
    code = (
        "import reduce_rank_buffers_amd._lib as L\n"
        f"L.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
        "import reduce_rank_buffers_amd.api as api\n"
        "try:\n"
        "    api.Plan(8, 64, 'bf16', api.PARTIAL, api.REPLICATED, 'reduce')\n"
        "except RuntimeError as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    raise SystemExit('no error')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([_sys.executable, "-c", code], cwd=root, capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "is not built" in res.stdout
