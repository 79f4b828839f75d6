"""GPU parity of the SNAC chains in the memory-model build (librrb_fenced.so:
flags published with agent-scope release stores, acquire fences after flags
are seen) against the oracle, through the C ABI: the All-Reduce chain
variants at decode payloads from 8 to 512 KiB per rank, late ranks that
force retries and cross the write-after-read guards, 8192 chained epochs,
and chains of other collectives.  The build must report its ordering and
refuse the flag-in-data chain."""

import sys

import numpy as np
import pytest
import torch

from oracle import chain as OC
from reduce_rank_buffers_amd import api, inputs
from reduce_rank_buffers_amd import _lib as L
from tests.gpu_util import DEV, require_gpu, to_dev
from tests.test_gpu_chain import R, _check_chain
from tests.test_gpu_plan_chain import _run_chain

pytestmark = pytest.mark.gpu

FENCED_VARIANTS = ["barrier", "dual", "speculative", "speculative_always", "twoshot"]
FENCED_SPEC_MAX_BYTES = 8 << 10  # that build's All-Reduce chains speculate up to this payload per rank


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _fenced_slices(ch):
    # the fenced build's default slices per rank: 64 vectors per workgroup,
    # up to 16 below 128 KiB per rank and 32 from there
    nvec = ch.count * 2 // 16
    return min(max(1, min(32 if nvec >= 8192 else 16, nvec // 64)), 2048 // R, nvec)


@pytest.fixture(scope="module", autouse=True)
def fenced_library():
    prev = L.select(True)
    assert L.lib().rrb_snac_fenced() == 1
    yield
    L.restore(prev)


@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_fenced_chain_variants_bit_exact(b):
    require_gpu()
    n, E = b * 4096, 64
    ins_np = inputs.chain(E, R, n)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    for v in FENCED_VARIANTS:
        _say(f"fenced chain b={b} h=4096 variant={v}")
        ch = api.SnacChain(R, n, "bf16", v)
        stats = torch.zeros(4, dtype=torch.int64, device=DEV)
        out = torch.empty_like(inp)
        ch.run(inp, out, stats=stats)
        ch.check()
        _check_chain(out, want, f"fenced {v} b={b}")
        st = stats.cpu().tolist()
        assert st[2] == 0
        assert st[3] == E * R * _fenced_slices(ch)
        if v == "speculative" and n * 2 > FENCED_SPEC_MAX_BYTES:
            assert st[0] == 0 and st[1] == 0  # waits for the flags first
        ch.close()


@pytest.mark.parametrize("v", ["barrier", "dual", "speculative", "twoshot"])
def test_fenced_chain_staggered(v):
    """Late ranks at 8 and 128 KiB per rank: retries and guards at skew."""
    require_gpu()
    for n in (4096, 65536):
        E = 32
        ins_np = inputs.chain(E, R, n, kind=84)
        want = OC.allreduce_chain(ins_np)
        inp = to_dev(ins_np)
        for st in ([r * 64 for r in range(R)], [0, 0, 0, 640, 0, 0, 0, 0]):
            _say(f"fenced stagger {v} n={n} {st}")
            ch = api.SnacChain(R, n, "bf16", v)
            stats = torch.zeros(4, dtype=torch.int64, device=DEV)
            out = torch.empty_like(inp)
            ch.run(inp, out, stats=stats, stagger=torch.tensor(st, dtype=torch.int32, device=DEV))
            ch.check()
            _check_chain(out, want, f"fenced stagger {v} n={n} {st}")
            s = stats.cpu().tolist()
            if v == "speculative" and n == 4096:
                assert s[0] > 0  # late ranks force the retry path
            ch.close()


@pytest.mark.parametrize("v", ["dual", "speculative", "twoshot"])
def test_fenced_8192_epochs_exact(v):
    """8192 chained All-Reduces over 256 seeded input sets at 8 KiB per rank,
    late ranks changing every call; every result bit-exact."""
    require_gpu()
    n, pool, total = 4096, 256, 8192
    ins_np = inputs.chain(pool, R, n, kind=85)
    want = np.stack(OC.allreduce_chain(ins_np))
    inp = to_dev(ins_np)
    want_dev = to_dev(np.repeat(want[:, None, :], R, axis=1))
    ch = api.SnacChain(R, n, "bf16", v)
    out = torch.empty_like(inp)
    rng = np.random.default_rng(86)
    done = 0
    while done < total:
        st = torch.from_numpy(rng.integers(0, 256, size=R).astype(np.int32)).to(DEV)
        ch.run(inp, out, stagger=st)
        if not torch.equal(out, want_dev):
            ch.check()
            bad = (out != want_dev).nonzero()
            raise AssertionError(f"fenced {v} mismatch after {done} epochs at {bad[:5].tolist()}")
        done += pool
    ch.check()
    _say(f"fenced {v}: {done} epochs exact")
    ch.close()


@pytest.mark.parametrize("name", ["all_reduce", "all_gather", "all_to_all", "reduce", "broadcast"])
@pytest.mark.parametrize("variant", ["barrier", "dual", "speculative"])
def test_fenced_plan_chains(name, variant):
    require_gpu()
    _say(f"fenced plan chain {name} {variant}")
    stats, ch = _run_chain(name, R, 8 * 1024, "bf16", variant, E=16)
    assert stats[2] == 0
    if variant == "speculative":
        assert stats[0] == 0 and stats[1] == 0  # that build's plan chains wait for the flags first
    ch.close()


def test_fenced_build_refuses_flag_in_data():
    require_gpu()
    with pytest.raises(L.RrbError) as e:
        api.SnacChain(R, 4096, "bf16", "lamport")
    assert e.value.status == L.RRB_EUNSUPPORTED
