"""GPU parity of the SNAC decode chain against the oracle, through the C ABI.

Each of the 64 epochs (32 layers x 2 All-Reduces) must give every rank the
exact oracle All-Reduce of that epoch's payloads, for the barrier,
dual-buffer, speculative, twoshot, flag-in-data and graph variants, at every
payload of the decode chain workload (b in 1..64 tokens x h in {4096, 8192}
bf16, N(0, 0.02)).  Protocol stress: staggered ranks (a test hook delays rank
r before every stage), the pages' own 100k-iteration exact-match check for
the speculative and flag-in-data variants, and a bounded wait forced to
expire from the host (tiny poll budget), which must end the kernel and report
RRB_ETIMEOUT rather than hang."""

import sys

import numpy as np
import pytest
import torch

from oracle import chain as OC
from reduce_rank_buffers_amd import api, inputs
from reduce_rank_buffers_amd import _lib as L
from tests.gpu_util import DEV, assert_bits_equal, from_dev, require_gpu, to_dev

pytestmark = pytest.mark.gpu

VARIANTS = ["barrier", "dual", "speculative", "speculative_always", "twoshot", "lamport", "graph"]
FLAG_VARIANTS = ["barrier", "dual", "speculative", "twoshot", "lamport"]
SPEC_MAX_BYTES = 128 << 10  # All-Reduce chains speculate up to this payload per rank
R = 8
EPOCHS = 64


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check_chain(out_dev, want, what):
    got = from_dev(out_dev.reshape(out_dev.shape[0], R, -1))
    for e in range(len(want)):
        for r in range(R):
            assert_bits_equal(got[e, r], want[e], f"{what} epoch {e} rank {r}")


@pytest.mark.parametrize("h", [4096, 8192])
@pytest.mark.parametrize("b", [1, 2, 4, 8, 16, 32, 64])
def test_chain_all_variants_bit_exact(b, h):
    require_gpu()
    n = b * h
    ins_np = inputs.chain(EPOCHS, R, n)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    for v in VARIANTS:
        _say(f"chain b={b} h={h} variant={v}")
        ch = api.SnacChain(R, n, "bf16", v)
        stats = torch.zeros(4, dtype=torch.int64, device=DEV)
        out = torch.empty_like(inp)
        ch.run(inp, out, stats=stats)
        ch.check()
        _check_chain(out, want, f"{v} b={b} h={h}")
        st = stats.cpu().tolist()
        assert st[2] == 0  # no timeouts
        if v != "graph":
            assert st[3] == EPOCHS * R * _slices_of(ch)
        if v == "speculative" and n * 2 > SPEC_MAX_BYTES:
            assert st[0] == 0 and st[1] == 0  # waits for the flags first: nothing to validate
        # a second call continues the epoch counter on the same flags
        out2 = torch.empty_like(inp)
        ch.run(inp, out2)
        ch.check()
        assert torch.equal(out2, out)


def _slices_of(ch):
    # the library's default slices per rank for a payload of nvec vectors
    nvec = ch.count * 2 // 16
    if ch.variant == "lamport":
        S = max(1, nvec // 64) if nvec < 4096 else min(256, nvec // 32) if nvec <= 16384 else 128
    else:
        S = 256 if nvec >= 32768 and ch.variant != "speculative_always" else max(1, min(128, nvec // 64))
    return min(S, 2048 // R, nvec)


@pytest.mark.parametrize("v", FLAG_VARIANTS)
def test_chain_staggered_ranks(v):
    """Late ranks (rank r sleeps about r x 4k cycles before each stage)."""
    require_gpu()
    n = 4096
    ins_np = inputs.chain(EPOCHS, R, n, kind=77)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    for pattern in ("ramp", "reverse", "one_slow"):
        if pattern == "ramp":
            st = [r * 64 for r in range(R)]
        elif pattern == "reverse":
            st = [(R - 1 - r) * 64 for r in range(R)]
        else:
            st = [0] * R
            st[5] = 400
        _say(f"stagger {v} {pattern}")
        stagger = torch.tensor(st, dtype=torch.int32, device=DEV)
        ch = api.SnacChain(R, n, "bf16", v)
        stats = torch.zeros(4, dtype=torch.int64, device=DEV)
        out = torch.empty_like(inp)
        ch.run(inp, out, stats=stats, stagger=stagger)
        ch.check()
        _check_chain(out, want, f"stagger {v} {pattern}")
        s = stats.cpu().tolist()
        if v == "speculative":
            _say(f"  misspec {s[0]} retries {s[1]}")
            assert s[0] > 0  # late ranks force the retry path
            # a failed check re-reads only the stale sources: at least one,
            # and never the workgroup's own rank
            assert s[0] <= s[1] <= s[0] * (R - 1)
        if v == "lamport":
            _say(f"  poll rounds {s[1]}")
            assert s[1] > 0  # late ranks leave untagged words to poll again


@pytest.mark.parametrize("n", [65536, 262144])
def test_chain_speculation_staggered_large(n):
    """Speculation forced at 128 KiB and 512 KiB per rank with late ranks: the
    first pass holds two vectors per lane, the rest of each slice follows in
    ordinary passes, and failed checks re-read the stale sources."""
    require_gpu()
    E = 12
    ins_np = inputs.chain(E, R, n, kind=81)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    stagger = torch.tensor([r * 64 for r in range(R)], dtype=torch.int32, device=DEV)
    _say(f"stagger speculative_always n={n}")
    ch = api.SnacChain(R, n, "bf16", "speculative_always")
    stats = torch.zeros(4, dtype=torch.int64, device=DEV)
    out = torch.empty_like(inp)
    ch.run(inp, out, stats=stats, stagger=stagger)
    ch.check()
    _check_chain(out, want, f"speculative_always n={n}")
    s = stats.cpu().tolist()
    _say(f"  misspec {s[0]} retries {s[1]}")
    assert s[2] == 0 and s[0] > 0 and s[0] <= s[1] <= s[0] * (R - 1)


@pytest.mark.parametrize("slices", [1, 3, 8])
def test_chain_slice_counts(slices):
    require_gpu()
    n = 8192
    ins_np = inputs.chain(16, R, n, kind=78)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    for v in VARIANTS:
        ch = api.SnacChain(R, n, "bf16", v, slices=slices)
        out = torch.empty_like(inp)
        ch.run(inp, out)
        ch.check()
        _check_chain(out, want, f"slices={slices} {v}")


def test_chain_other_rank_counts_and_fp32():
    require_gpu()
    for Rx, n, dt in [(2, 4096, "bf16"), (3, 1024, "bf16"), (16, 2048, "bf16"), (8, 2048, "f32"),
                      (8, 800, "bf16"), (5, 4000, "bf16")]:
        E = 8
        rng = np.random.default_rng(Rx * n)
        if dt == "bf16":
            ins_np = inputs.chain(E, Rx, n, kind=79)
        else:
            ins_np = rng.standard_normal((E, Rx, n)).astype(np.float32)
        want = OC.allreduce_chain(ins_np, dt)
        inp = to_dev(ins_np)
        for v in VARIANTS:
            _say(f"chain R={Rx} n={n} {dt} {v}")
            ch = api.SnacChain(Rx, n, dt, v)
            out = torch.empty_like(inp)
            ch.run(inp, out)
            ch.check()
            got = from_dev(out)
            for e in range(E):
                for r in range(Rx):
                    assert_bits_equal(got[e, r], want[e], f"R={Rx} {dt} {v} e={e} r={r}")


@pytest.mark.parametrize("v", FLAG_VARIANTS)
def test_100k_iterations_exact(v):
    """The pages' correctness check for speculative reduction: 100k chained
    All-Reduces, every result bit-exact (here against precomputed oracle
    results; payloads cycle through 256 seeded input sets, so a value left
    from an earlier epoch shows as a mismatch).  Run for every variant."""
    require_gpu()
    n, pool, per_call, total = 4096, 256, 256, 100_000
    ins_np = inputs.chain(pool, R, n, kind=80)
    want = np.stack(OC.allreduce_chain(ins_np))  # [pool, n]
    inp = to_dev(ins_np)
    want_dev = to_dev(np.repeat(want[:, None, :], R, axis=1))  # [pool, R, n]
    ch = api.SnacChain(R, n, "bf16", v)
    stats = torch.zeros(4, dtype=torch.int64, device=DEV)
    out = torch.empty_like(inp)
    done = 0
    calls = 0
    while done < total:
        ch.run(inp, out, stats=stats)
        if not torch.equal(out, want_dev):
            ch.check()
            bad = (out != want_dev).nonzero()
            raise AssertionError(f"{v} mismatch after {done} epochs at {bad[:5].tolist()}")
        done += per_call
        calls += 1
        if calls % 100 == 0:
            _say(f"  {done} epochs exact")
    ch.check()
    s = stats.cpu().tolist()
    _say(f"100k {v}: misspec {s[0]} retries {s[1]} epochs {done}")


@pytest.mark.parametrize("v", ["speculative", "lamport"])
def test_100k_staggered_exact(v):
    """100k chained All-Reduces with late ranks that change every call
    (seeded delays of 0-255 sleeps per rank before each stage), so the
    speculative check fails and retries, and flag-in-data polls find
    untagged words, throughout; every result bit-exact."""
    require_gpu()
    n, pool, per_call, total = 4096, 256, 256, 100_000
    ins_np = inputs.chain(pool, R, n, kind=82)
    want = np.stack(OC.allreduce_chain(ins_np))
    inp = to_dev(ins_np)
    want_dev = to_dev(np.repeat(want[:, None, :], R, axis=1))
    ch = api.SnacChain(R, n, "bf16", v)
    stats = torch.zeros(4, dtype=torch.int64, device=DEV)
    out = torch.empty_like(inp)
    rng = np.random.default_rng(83)
    done = 0
    while done < total:
        st = rng.integers(0, 256, size=R).astype(np.int32)
        stagger = torch.from_numpy(st).to(DEV)
        ch.run(inp, out, stats=stats, stagger=stagger)
        if not torch.equal(out, want_dev):
            ch.check()
            bad = (out != want_dev).nonzero()
            raise AssertionError(f"{v} mismatch after {done} epochs, stagger {st.tolist()}: {bad[:5].tolist()}")
        done += per_call
        if done % 25600 == 0:
            _say(f"  {done} staggered epochs exact")
    ch.check()
    s = stats.cpu().tolist()
    _say(f"100k staggered {v}: misspec {s[0]} retries {s[1]}")
    assert s[2] == 0
    assert s[1] > 0  # retries (speculative) or poll rounds (flag-in-data) happened


@pytest.mark.parametrize("v", ["barrier", "dual", "speculative", "twoshot"])
def test_many_slices_stress_exact(v):
    """128 KiB payloads take 128 workgroups per rank (1024 in all) for the
    flag variants: 8192 chained All-Reduces over 32 seeded input sets, every
    result bit-exact."""
    require_gpu()
    n, pool, total = 65536, 32, 8192
    ins_np = inputs.chain(pool, R, n, kind=82)
    want = np.stack(OC.allreduce_chain(ins_np))
    inp = to_dev(ins_np)
    want_dev = to_dev(np.repeat(want[:, None, :], R, axis=1))
    ch = api.SnacChain(R, n, "bf16", v)
    out = torch.empty_like(inp)
    done = 0
    while done < total:
        ch.run(inp, out)
        if not torch.equal(out, want_dev):
            ch.check()
            bad = (out != want_dev).nonzero()
            raise AssertionError(f"{v} mismatch after {done} epochs at {bad[:5].tolist()}")
        done += pool
    ch.check()
    _say(f"many-slices {v}: {done} epochs exact")


@pytest.mark.parametrize("v", ["barrier", "dual", "speculative", "twoshot", "lamport"])
def test_many_slices_staggered_exact(v):
    """128 KiB payloads (128 workgroups per rank) with late ranks: rank r
    sleeps about r x 4k cycles, or rank 3 about 40k, before every stage, so
    the write-after-read guards are crossed at skew; every epoch bit-exact."""
    require_gpu()
    n, E = 65536, 32
    ins_np = inputs.chain(E, R, n, kind=83)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    for st in ([r * 64 for r in range(R)], [0, 0, 0, 640, 0, 0, 0, 0]):
        ch = api.SnacChain(R, n, "bf16", v)
        out = torch.empty_like(inp)
        ch.run(inp, out, stagger=torch.tensor(st, dtype=torch.int32, device=DEV))
        ch.check()
        _check_chain(out, want, f"many slices staggered {v} {st}")


def test_bounded_wait_times_out_cleanly():
    """A poll budget of 1 with one rank delayed: waits expire, every
    workgroup leaves, and the host gets RRB_ETIMEOUT (no hang)."""
    require_gpu()
    n = 4096
    ins_np = inputs.chain(4, R, n, kind=81)
    inp = to_dev(ins_np)
    st = [0] * R
    st[7] = 20000
    stagger = torch.tensor(st, dtype=torch.int32, device=DEV)
    for v in ("barrier", "dual", "twoshot", "lamport"):
        ch = api.SnacChain(R, n, "bf16", v)
        stats = torch.zeros(4, dtype=torch.int64, device=DEV)
        out = torch.empty_like(inp)
        ch.run(inp, out, stats=stats, stagger=stagger, spin_limit=1)
        with pytest.raises(L.RrbError) as e:
            ch.check()
        assert e.value.status == L.RRB_ETIMEOUT
        assert stats.cpu().tolist()[2] > 0


def test_graph_chain_replays_and_rebuilds():
    """The graph variant caches its HIP graph per (in, out, epochs): replays
    with new input contents (eager copies and synchronisations between the
    replays) and a rebuild for new buffers all stay bit-exact."""
    require_gpu()
    n, E = 4096, 16
    ch = api.SnacChain(R, n, "bf16", "graph")
    inp = torch.empty((E, R, n), dtype=torch.int16, device=DEV)
    out = torch.empty_like(inp)
    for k in range(3):
        host = inputs.chain(E, R, n, kind=90 + k)
        inp.copy_(to_dev(host))
        torch.cuda.synchronize()
        ch.run(inp, out)
        ch.check()
        _check_chain(out, OC.allreduce_chain(host), f"graph replay {k}")
    inp2 = to_dev(inputs.chain(8, R, n, kind=95))
    out2 = torch.empty_like(inp2)
    ch.run(inp2, out2)
    ch.check()
    _check_chain(out2, OC.allreduce_chain(inputs.chain(8, R, n, kind=95)), "graph rebuild")
    with pytest.raises(L.RrbError):
        ch.run(inp, out, stagger=torch.zeros(R, dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("v", ["dual", "lamport", "graph"])
def test_bound_chain_call_matches_oracle(v):
    """A chain call marshalled once and issued twice: both bit-exact, and the
    epoch counter carries across the calls."""
    require_gpu()
    n = 8192
    ins_np = inputs.chain(EPOCHS, R, n, kind=82)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    out = torch.empty_like(inp)
    ch = api.SnacChain(R, n, "bf16", v)
    call = ch.bound(inp, out)
    for k in range(2):
        out.zero_()
        call()
        ch.check()
        _check_chain(out, want, f"bound {v} call {k}")


@pytest.mark.parametrize("v", FLAG_VARIANTS)
def test_chain_cooperative_launch(v):
    """RRB_SNAC_COOPERATIVE: the same chain through a cooperative launch (the
    default takes a plain launch when the grid fits the device)."""
    require_gpu()
    n = 4096
    ins_np = inputs.chain(16, R, n, kind=83)
    want = OC.allreduce_chain(ins_np)
    inp = to_dev(ins_np)
    out = torch.empty_like(inp)
    ch = api.SnacChain(R, n, "bf16", v, cooperative=True)
    ch.run(inp, out)
    ch.check()
    _check_chain(out, want, f"cooperative {v}")
