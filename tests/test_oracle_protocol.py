"""Stage / notify / consume protocol model (CPU only).

Checks, over seeded random schedules with and without a slow rank:
* the barrier and dual-buffer variants always produce the exact sums;
* removing the bottom barrier without a second buffer breaks results (the
  write-after-read hazard the bottom barrier exists for);
* the speculative variant with the pages' load order (payload, then flag)
  can validate a stale read, and every such wrong result coincides with a
  source overtaking the reader between its payload read and its flag read
  (the load-bearing premise);
* issuing the flag loads before the payload loads makes every validated
  result exact under sequential consistency;
* no flag ever runs ahead of the epoch being validated (so the reduced flag
  equals R * epoch exactly when every flag does).
"""

import random

import pytest

from oracle import protocol as P


def _sweep(variant, R, E, L, seeds, bias=None):
    rng = random.Random(1000 * R + E)
    wrong = unexplained = misspec = overrun = 0
    for seed in range(seeds):
        inp = [[[rng.randint(-9, 9) for _ in range(L)] for _ in range(R)] for _ in range(E)]
        out, st = P.run(variant, inp, seed=seed, bias=bias)
        exp = P.expected(inp)
        for e in range(E):
            for r in range(R):
                if out[e][r] != exp[e]:
                    wrong += 1
                    if (e + 1, r) not in st["overtaken_at"]:
                        unexplained += 1
        misspec += st["misspec"]
        overrun += st["overrun"]
    return wrong, unexplained, misspec, overrun


BIASES = [None, "slow_last"]


def _bias(b, R):
    return None if b is None else [1.0] * (R - 1) + [0.15]


@pytest.mark.parametrize("variant", ["barrier", "dual", "speculative_ff"])
@pytest.mark.parametrize("R", [2, 3])
@pytest.mark.parametrize("b", BIASES)
def test_sound_variants_always_exact(variant, R, b):
    wrong, _, misspec, overrun = _sweep(variant, R, 5, 2, 200, _bias(b, R))
    assert wrong == 0
    assert overrun == 0
    if variant == "speculative_ff":
        assert misspec > 0  # the retry path is exercised


def test_missing_bottom_barrier_exhibits_hazard():
    wrong, *_ = _sweep("nobottom", 3, 5, 2, 200)
    assert wrong > 0


@pytest.mark.parametrize("b", BIASES)
def test_payload_first_speculation_fails_only_by_overtaking(b):
    wrong, unexplained, misspec, overrun = _sweep("speculative", 3, 5, 2, 300, _bias(b, 3))
    assert wrong > 0          # the premise can be violated by a schedule
    assert unexplained == 0   # ... and only that way
    assert overrun == 0
    assert misspec > 0


def _sweep_tagged(variant, R, E, L, seeds, bias=None, tag_mod=1 << 16):
    """(wrong results, deadlocked schedules) over seeded schedules."""
    rng = random.Random(77 * R + E + L)
    wrong = deadlocks = 0
    for seed in range(seeds):
        inp = [[[rng.randint(-9, 9) for _ in range(L)] for _ in range(R)] for _ in range(E)]
        try:
            out, _ = P.run(variant, inp, seed=seed, bias=bias, tag_mod=tag_mod)
        except RuntimeError:
            deadlocks += 1
            continue
        exp = P.expected(inp)
        wrong += sum(out[e][r] != exp[e] for e in range(E) for r in range(R))
    return wrong, deadlocks


@pytest.mark.parametrize("R", [2, 3])
@pytest.mark.parametrize("b", BIASES)
@pytest.mark.parametrize("tag_mod", [3, 1 << 16])
def test_flag_in_data_dual_buffer_always_exact(R, b, tag_mod):
    """Tagged words, no flags, no ordering between words: exact and live."""
    wrong, deadlocks = _sweep_tagged("lamport", R, 6, 3, 200, _bias(b, R), tag_mod)
    assert (wrong, deadlocks) == (0, 0)


def test_flag_in_data_needs_tags_that_tell_e_from_e_minus_2():
    """With the tag taken modulo 2 a stale word of epoch e - 2 in the same
    buffer carries the tag of epoch e and is accepted."""
    wrong, deadlocks = _sweep_tagged("lamport", 3, 6, 3, 200, [1.0, 1.0, 0.15], tag_mod=2)
    assert deadlocks == 0
    assert wrong > 0


def test_flag_in_data_single_buffer_exhibits_hazard():
    """One tagged buffer: a fast rank's next epoch overwrites words a slow
    reader still wants, which ends in a wrong result or a wait that never
    ends."""
    wrong, deadlocks = _sweep_tagged("lamport_single", 3, 6, 3, 200, [1.0, 1.0, 0.15])
    assert wrong + deadlocks > 0
