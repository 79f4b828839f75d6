"""Step model of stage / notify / consume for a chain of All-Reduces (oracle;
test infrastructure only).

Purlin: Separating Orchestration from the Datapath of Collectives ("The Purlin
PDF describes a three-layer design") names the orchestration layer Stage,
Notify, And Consume.  SiFAR: Synchronization-Free All-Reduce for Low-Latency
LLM Inference (review page: abstract; Fig. 1, Fig. 8, Fig. 14; "Load-bearing
premise"; referee report on §8.1) gives the variants modelled here:

``barrier``      one staging buffer, a top barrier (wait for every rank's
                 flag) before reading and a bottom barrier (wait until every
                 rank has finished reading) before the next stage -- the
                 bottom barrier guards the write-after-read hazard.
``nobottom``     one buffer, top barrier only -- *unsafe*: exhibits the
                 hazard the bottom barrier exists for.
``dual``         two staging buffers alternating by epoch parity, top barrier
                 only: the next epoch's top barrier already proves every
                 reader of this buffer is done, so no bottom barrier.
``speculative``  dual buffers, no top barrier: read the payload first, then
                 reduce the per-rank validation flags and compare the sum with
                 R * epoch; on mismatch wait for the flags and read again.
``speculative_ff``  the same, but the flag loads are issued *before* the
                 payload loads (with no wait between them).  Under sequential
                 consistency this is always correct: a flag equal to the
                 epoch proves the source finished staging before the payload
                 reads began.  On hardware the remaining premise is only that
                 a later-issued load is not served earlier than a flag load
                 by more than the writer's stage-to-flag gap.

``lamport``      flag-in-data, the Lamport-style All-Reduce SiFAR compares
                 against (review page, Fig. 20): no flags at all.  Every
                 payload word is stored together with a tag, the epoch modulo
                 ``tag_mod``, in one single-copy-atomic access, and a reader
                 polls each word until it carries the tag of the epoch it
                 wants.  Words are stored and read in a random order per rank
                 and epoch, since nothing orders one word against another.
                 Two buffers alternate by epoch parity: a rank overwrites
                 buffer e % 2 at epoch e + 2 only after it has read every
                 rank's epoch e + 1 words, which each rank stored after its
                 own epoch-e reads.  Sound when tag_mod >= 3 (the tags of e
                 and e - 2 differ, and the initial tag 0 only meets epochs
                 that already overwrote it).
``lamport_single``  the same with one buffer -- *unsafe*: a fast rank's next
                 epoch overwrites words a slow reader has not read yet.

Each rank is a generator that performs one shared-memory access per step;
``run`` interleaves ranks under a seeded scheduler, so every schedule is a
sequentially consistent execution.  Payloads are small integers, so a wrong
result is an exact mismatch.  For ``speculative`` the model also records, for
every validated read, whether some source *overtook* the reader -- published
its flag after the reader's first payload read of it and before the reader's
flag read -- which is exactly the premise the pages rely on.
"""

import random

VARIANTS = ("barrier", "nobottom", "dual", "speculative", "speculative_ff", "lamport",
            "lamport_single")


def _nbuf(variant):
    return 1 if variant in ("barrier", "nobottom", "lamport_single") else 2


class _Mem:
    def __init__(self, R, L, nbuf):
        self.staging = [[[0] * L for _ in range(R)] for _ in range(nbuf)]
        # flag-in-data words: (tag, value), stored and read as one access
        self.tagged = [[[(0, 0)] * L for _ in range(R)] for _ in range(nbuf)]
        self.flag = [[0] * R for _ in range(nbuf)]
        self.done = [0] * R
        self.clock = 0
        self.notify_time = {}  # (rank, epoch) -> clock of the flag store


def _rank_tagged(mem, r, R, L, inputs, out, tag_mod, order_rng, nbuf):
    """Flag-in-data rank: every word carries its epoch's tag."""
    E = len(inputs)
    for e in range(1, E + 1):
        b = e % nbuf
        tag = e % tag_mod
        # Stage: one (tag, value) store per word, in no particular order.
        for i in order_rng.sample(range(L), L):
            mem.tagged[b][r][i] = (tag, inputs[e - 1][r][i])
            yield None
        # Consume: poll each word of each source until its tag is this
        # epoch's; the check and the read are the same access.
        got = [[None] * L for _ in range(R)]
        cells = [(s, i) for s in range(R) for i in range(L)]
        for s, i in order_rng.sample(cells, len(cells)):
            yield lambda s=s, i=i: mem.tagged[b][s][i][0] == tag
            got[s][i] = mem.tagged[b][s][i][1]
        out[e - 1][r] = [sum(got[s][i] for s in range(R)) for i in range(L)]


def _rank(mem, variant, r, R, L, inputs, out, stats):
    nbuf = _nbuf(variant)
    E = len(inputs)
    for e in range(1, E + 1):
        b = e % nbuf
        # Stage: the rank's payload lands in its staged buffer, word by word.
        for i in range(L):
            mem.staging[b][r][i] = inputs[e - 1][r][i]
            yield None
        # Notify.
        mem.flag[b][r] = e
        mem.notify_time[(r, e)] = mem.clock
        yield None
        first_read = {}
        if not variant.startswith("speculative"):
            # Consume-wait: the top barrier.
            yield lambda: all(mem.flag[b][s] >= e for s in range(R))
            acc = [0] * L
            for s in range(R):
                for i in range(L):
                    acc[i] += mem.staging[b][s][i]
                    yield None
        else:
            flag_read = {}
            total = 0

            def read_flags():
                nonlocal total
                for s in range(R):
                    f = mem.flag[b][s]
                    flag_read[s] = mem.clock
                    if f > e:
                        stats["overrun"] += 1
                    total += f
                    yield None

            def read_payload():
                for s in range(R):
                    first_read[s] = mem.clock
                    for i in range(L):
                        acc[i] += mem.staging[b][s][i]
                        yield None

            acc = [0] * L
            if variant == "speculative":
                # The pages' order: payload first, then the reduced flag.
                yield from read_payload()
                yield from read_flags()
            else:
                # Flags issued first, payload right after, no wait between.
                yield from read_flags()
                yield from read_payload()
            if total != R * e:
                stats["misspec"] += 1
                yield lambda: all(mem.flag[b][s] >= e for s in range(R))
                acc = [0] * L
                for s in range(R):
                    for i in range(L):
                        acc[i] += mem.staging[b][s][i]
                        yield None
            else:
                for s in range(R):
                    t = mem.notify_time.get((s, e))
                    if t is not None and first_read[s] <= t < flag_read[s]:
                        stats["overtaken"] += 1
                        stats["overtaken_at"].add((e, r))
                        break
        out[e - 1][r] = acc
        if variant == "barrier":
            mem.done[r] = e
            yield None
            yield lambda: all(mem.done[s] >= e for s in range(R))


def run(variant, inputs, seed=0, bias=None, tag_mod=1 << 16):
    """Run one schedule.  inputs[e][r] is a list of L ints.

    ``bias``: optional list of per-rank weights for the scheduler (a slow rank
    gets a small weight), standing in for staggered starts.  ``tag_mod``: the
    modulus of the flag-in-data tags (the GPU uses 16-bit tags).
    Returns (outputs[e][r], stats).  A schedule in which every live rank waits
    forever raises RuntimeError.
    """
    if variant not in VARIANTS:
        raise ValueError(variant)
    E = len(inputs)
    R = len(inputs[0])
    L = len(inputs[0][0])
    nbuf = _nbuf(variant)
    mem = _Mem(R, L, nbuf)
    out = [[None] * R for _ in range(E)]
    stats = {"misspec": 0, "overrun": 0, "overtaken": 0, "steps": 0,
             "overtaken_at": set()}
    if variant.startswith("lamport"):
        gens = [_rank_tagged(mem, r, R, L, inputs, out, tag_mod,
                             random.Random(seed * 7919 + r), nbuf) for r in range(R)]
    else:
        gens = [_rank(mem, variant, r, R, L, inputs, out, stats) for r in range(R)]
    waiting = [None] * R
    live = set(range(R))
    rng = random.Random(seed)
    weights = bias or [1.0] * R
    while live:
        ready = [r for r in live if waiting[r] is None or waiting[r]()]
        if not ready:
            raise RuntimeError("deadlock in protocol model")
        r = rng.choices(ready, weights=[weights[x] for x in ready])[0]
        waiting[r] = None
        try:
            w = next(gens[r])
        except StopIteration:
            live.discard(r)
            continue
        mem.clock += 1
        stats["steps"] += 1
        if callable(w):
            waiting[r] = w
    return out, stats


def expected(inputs):
    """Exact per-epoch sums: what every rank must hold after each epoch."""
    return [[sum(col) for col in zip(*ins)] for ins in inputs]
