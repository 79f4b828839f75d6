"""The Python binding rejects buffers the library would read or write out of
bounds, before any call into librrb: wrong element types, strided views,
undersized buffers, missing ranks, tensors off the GPU, malformed chain and
routing arrays.  Runs on the CPU (the library is loaded; nothing launches):
every check before the device check is reached with CPU tensors, and the
device check itself with a well-formed CPU tensor."""

import pytest
import torch

from reduce_rank_buffers_amd import api


@pytest.fixture
def ar_plan(librrb):
    return api.Plan(8, 64, "bf16", api.PARTIAL, api.REPLICATED, "reduce")


def _bufs(n, dtype=torch.bfloat16, R=8):
    return [torch.zeros(n, dtype=dtype) for _ in range(R)]


def test_dtype_of_accepts_only_bf16_patterns_and_f32():
    assert api._dtype_of(torch.zeros(2, dtype=torch.bfloat16)) == api.L.RRB_BF16
    assert api._dtype_of(torch.zeros(2, dtype=torch.int16)) == api.L.RRB_BF16
    assert api._dtype_of(torch.zeros(2, dtype=torch.float32)) == api.L.RRB_F32
    for bad in (torch.float16, torch.int32, torch.float64, torch.uint8):
        with pytest.raises(ValueError):
            api._dtype_of(torch.zeros(2, dtype=bad))


def test_collective_rejects_fp16(librrb):
    with pytest.raises(ValueError):
        api.all_reduce(_bufs(64, torch.float16), _bufs(64, torch.float16))


PLAN_CASES = {"dtype": "is not bfloat16", "strided": "not contiguous", "short": "at least 64",
              "missing": "needs a buffer", "too_many": "at most 8", "device": "not on the current GPU"}


@pytest.mark.parametrize("case", list(PLAN_CASES))
def test_plan_run_rejects(ar_plan, case):
    ins, outs = _bufs(64), _bufs(64)
    if case == "dtype":
        ins[3] = torch.zeros(64, dtype=torch.float32)
    elif case == "strided":
        outs[5] = torch.zeros(128, dtype=torch.bfloat16)[::2]
    elif case == "short":
        ins[7] = torch.zeros(63, dtype=torch.bfloat16)
    elif case == "missing":
        outs = outs[:7]
    elif case == "too_many":
        ins = ins + [torch.zeros(64, dtype=torch.bfloat16)]
    with pytest.raises(ValueError) as e:
        ar_plan.run(ins, outs)  # 'device': well formed, but on the CPU
    assert PLAN_CASES[case] in str(e.value)


def test_bound_checks_at_construction(ar_plan):
    ins, outs = _bufs(64), _bufs(64)
    outs[2] = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(ValueError) as e:
        api.Bound(ar_plan, ins, outs)
    assert "outs[2]" in str(e.value)


def test_root_plans_take_none_for_unwritten_ranks(librrb):
    p = api.Plan(8, 64, "bf16", api.PARTIAL, (api.L.RRB_ROOT, 2), "reduce")
    outs = [None, None, torch.zeros(64, dtype=torch.bfloat16)] + [None] * 5
    with pytest.raises(ValueError) as e:
        p.run(_bufs(64), outs)
    assert "not on the current GPU" in str(e.value)  # only the device check is left
    outs[2] = torch.zeros(32, dtype=torch.bfloat16)
    with pytest.raises(ValueError) as e:
        p.run(_bufs(64), outs)
    assert "at least 64" in str(e.value)


def test_weights_only_on_combine_plans(ar_plan, librrb):
    w = torch.zeros(8, dtype=torch.float32)
    cp = api.Plan(8, 64, "bf16", api.SHARD, api.REPLICATED, "copy")
    for p in (cp, ar_plan):
        with pytest.raises(ValueError) as e:
            p.run(_bufs(64), _bufs(64), weights=w)
        assert "combine plans only" in str(e.value)


def _bare(cls, **attrs):
    """An instance without its GPU-allocating constructor, for the checks."""
    o = cls.__new__(cls)
    o.handle = None
    for k, v in attrs.items():
        setattr(o, k, v)
    return o


CHAIN_CASES = {"rank_dim": "shape [epochs, 8, 4096]", "stride": "shape [epochs, 8, 4096]",
               "epochs": "different numbers of epochs", "dtype": "is not bfloat16",
               "strided": "shape [epochs, 8, 4096]", "strided_full": "not contiguous",
               "stats": "torch.int64", "stats_short": "at least 4", "stagger": "at least 8",
               "device": "not on the current GPU"}


@pytest.mark.parametrize("case", list(CHAIN_CASES))
def test_chain_buffers_rejected(case):
    ch = _bare(api.SnacChain, nranks=8, strides=(4096, 4096), dtype=api.L.RRB_BF16)
    E = 4
    inp = torch.zeros(E, 8, 4096, dtype=torch.int16)
    out = torch.zeros(E, 8, 4096, dtype=torch.int16)
    stats = stagger = None
    if case == "rank_dim":
        inp = torch.zeros(E, 7, 4096, dtype=torch.int16)
    elif case == "stride":
        out = torch.zeros(E, 8, 4095, dtype=torch.int16)
    elif case == "epochs":
        out = torch.zeros(E + 1, 8, 4096, dtype=torch.int16)
    elif case == "dtype":
        inp = torch.zeros(E, 8, 4096, dtype=torch.float32)
    elif case == "strided":
        inp = torch.zeros(E, 8, 8192, dtype=torch.int16)[:, :, ::2][:, :, :4095]
    elif case == "strided_full":
        inp = torch.zeros(E, 8, 8192, dtype=torch.int16)[:, :, ::2]
    elif case == "stats":
        stats = torch.zeros(4, dtype=torch.int32)
    elif case == "stats_short":
        stats = torch.zeros(3, dtype=torch.int64)
    elif case == "stagger":
        stagger = torch.zeros(7, dtype=torch.int32)
    with pytest.raises(ValueError) as e:
        ch.check_buffers(inp, out, stats, stagger)
    assert CHAIN_CASES[case] in str(e.value)


def test_plan_chain_strides_checked():
    ch = _bare(api.SnacPlanChain, nranks=8, strides=(256, 2048), dtype=api.L.RRB_BF16)
    with pytest.raises(ValueError) as e:
        ch.check_buffers(torch.zeros(2, 8, 2048, dtype=torch.int16),
                         torch.zeros(2, 8, 2048, dtype=torch.int16))
    assert "[epochs, 8, 256]" in str(e.value)


ROUTE_CASES = {"idx_dtype": "topk_idx: expected a tensor of torch.int32",
               "w_dtype": "topk_w: expected a tensor of torch.float32",
               "short": "at least 512", "offsets": "at least 9", "missing": "required",
               "device": "not on the current GPU"}


@pytest.mark.parametrize("case", list(ROUTE_CASES))
def test_route_arrays_rejected(case):
    p = _bare(api.MoeDevicePlan, nranks=8, tokens=64, topk=8, _lib=None)
    idx = torch.zeros(64, 8, dtype=torch.int32)
    w = torch.zeros(64, 8, dtype=torch.float32)
    offs = None
    if case == "idx_dtype":
        idx = idx.to(torch.int64)
    elif case == "w_dtype":
        w = w.to(torch.bfloat16)
    elif case == "short":
        idx = torch.zeros(63, 8, dtype=torch.int32)
    elif case == "offsets":
        offs = torch.zeros(8, dtype=torch.int32)
    elif case == "missing":
        w = None
    with pytest.raises(ValueError) as e:
        p.route(idx, w, offs)
    assert ROUTE_CASES[case] in str(e.value)
