"""Pins for the oracle's bf16 conversions (CPU only).

The oracle rounds by comparing distances in float64; these tests pin it to
(1) hand cases from the IEEE 754 definition of roundTiesToEven
(tests/golden/bf16_rne_cases.txt), and (2) torch's CPU float->bfloat16 cast, a
library round-to-nearest-even, over a structured sweep that visits every
bf16 pattern with the low halves that decide ties.
"""

import os

import numpy as np
import torch

from oracle import bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rne_cases.txt")


def _torch_rne(u32):
    f = torch.from_numpy(np.asarray(u32, dtype=np.uint32).view(np.float32).copy())
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _load_golden():
    rows = []
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b, *_ = line.split()
            rows.append((int(a, 16), int(b, 16)))
    return rows


def test_golden_cases():
    rows = _load_golden()
    assert len(rows) >= 20
    x = np.array([a for a, _ in rows], dtype=np.uint32).view(np.float32)
    got = bf16.rne(x)
    for (a, b), g in zip(rows, got):
        assert int(g) == b, f"{a:08X}: got {int(g):04X}, want {b:04X}"


def test_structured_sweep_matches_torch():
    hi = np.arange(1 << 16, dtype=np.uint32) << np.uint32(16)
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF,
                     0xFFFE, 0xFFFF], dtype=np.uint32)
    u = (hi[:, None] | lows[None, :]).reshape(-1)
    x = u.view(np.float32)
    got = bf16.rne(x)
    want = _torch_rne(u)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0x7FC0)


def test_random_patterns_match_torch():
    rng = np.random.default_rng(7)
    u = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    got = bf16.rne(x)
    want = _torch_rne(u)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all(got[nan] == 0x7FC0)


def test_widen_is_exact_and_inverse():
    b = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16.widen(b)
    assert np.array_equal(f.view(np.uint32) >> np.uint32(16), b.astype(np.uint32))
    assert np.all((f.view(np.uint32) & np.uint32(0xFFFF)) == 0)
    back = bf16.rne(f)
    finite = ~np.isnan(f)
    assert np.array_equal(back[finite], b[finite])
