"""Helpers for the GPU parity tests: numpy <-> device, sentinels, and the
oracle applied in contiguous ranges for full-size compares."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

DEV = torch.device("cuda", 0)


# bf16 bit patterns for special-value tests: zeros, subnormals, ones, the
# largest finite values, infinities, and NaNs of both signs with and without
# payload (quiet and signalling).  Every NaN result must come out as 0x7FC0.
BF16_SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0002, 0x8003, 0x007F, 0x0080, 0x3F80,
                          0xBF80, 0x7F7F, 0xFF7F, 0x7F00, 0x4000, 0xC000, 0x3F81, 0xBF81, 0x0100,
                          0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7FC1, 0x7F81, 0xFF81], dtype=np.uint16)


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X (run them with -m gpu where one is present)"


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def from_dev(t):
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        return a.view(np.uint16)
    return a


def empty_like_np(n, dtype, fill=None):
    tdt = torch.int16 if dtype in ("bf16", np.uint16) else torch.float32
    t = torch.empty(int(n), dtype=tdt, device=DEV)
    if fill is not None:
        t.fill_(fill)
    return t


def sentinel(dtype):
    return -21555 if dtype == "bf16" else -12345.0  # 0xABCD as int16


def assert_bits_equal(got, want, what=""):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    g = got.view(np.uint8)
    w = want.view(np.uint8)
    if not np.array_equal(g, w):
        gi = got.view(np.uint16 if got.dtype.itemsize == 2 else np.uint32)
        wi = want.view(np.uint16 if want.dtype.itemsize == 2 else np.uint32)
        bad = np.nonzero(gi != wi)[0]
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {bad[:5]}: "
                             f"got {gi[bad[:5]]} want {wi[bad[:5]]}")


def oracle_elementwise(fn, ins, chunk=1 << 22):
    """fn (an elementwise oracle function of R equal-length arrays, such as
    oracle.fold.reduce) applied to contiguous element ranges in a thread pool,
    the results joined.  The oracle itself is unchanged: an elementwise
    definition gives the same bits on any split of the range.  Threads: the
    host's CPU share, at most 16."""
    n = len(ins[0])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    out = None

    def part(a):
        b = min(n, a + chunk)
        return a, fn([x[a:b] for x in ins])

    with ThreadPoolExecutor(max_workers=max(1, min(16, cores))) as pool:
        for a, r in pool.map(part, range(0, n, chunk)):
            if out is None:
                out = np.empty(n, dtype=r.dtype)
            out[a:a + len(r)] = r
    return out
