"""CPU oracle for the collective datapath -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``reduce_rank_buffers_amd`` and its HIP library) never imports, links or
calls it, and this package imports nothing from the product path.  Inputs
reach both sides as plain numpy arrays produced by the seeded generators in
``reduce_rank_buffers_amd.inputs``, which hold none of the method's
arithmetic.

What it computes, and where the pages define it:

* ``bf16``        -- widening bf16 -> fp32 and round-to-nearest-even fp32 ->
                     bf16, written from the definition of "nearest, ties to
                     even" (distance comparison in float64), not from a bit
                     trick.
* ``fold``        -- the Atom *reduce* primitive (Purlin: Separating
                     Orchestration from the Datapath of Collectives, "The
                     Purlin PDF describes a three-layer design"): an
                     elementwise sum over the R rank payloads, accumulated in
                     fp32 in fixed rank order 0..R-1, rounded once to bf16.
* ``collectives`` -- a collective as a naming of an input layout and an
                     output layout plus copy or reduce (same page and
                     section), and the seven named collectives written out
                     from their plain definitions (All-Reduce as in SiFAR:
                     Synchronization-Free All-Reduce for Low-Latency LLM
                     Inference, abstract and Fig. 5; twoshot's reduce-scatter
                     and all-gather halves, Fig. 6 and Fig. 9).
* ``moe``         -- expert-parallel dispatch (row copy by an expert index
                     map) and combine (weighted reduce in fixed ascending
                     expert order).
* ``chain``       -- the decode chain: each epoch's result is the All-Reduce
                     of that epoch's R payloads, whatever the orchestration
                     variant (SiFAR review, referee report on §8.1: the
                     speculative All-Reduce must match the barrier one
                     exactly).
* ``protocol``    -- a step-by-step model of stage / notify / consume with
                     barrier, dual-buffer and speculative variants, used to
                     exhibit the interleavings the speculative variant
                     depends on (SiFAR review, "Load-bearing premise").

Pins (checked by ``tests/test_oracle_*.py`` under ``-m "not gpu"``): torch's
CPU float->bfloat16 conversion and hand-picked tie cases for the rounding; an
exact rational emulation of IEEE binary32 addition for the fold; closed forms
(R = 1, equal ranks, cancelling pairs, small integers); the recursive
summation error bound; brute-force per-element loops for every layout map;
invariants (all-gather after reduce-scatter equals all-reduce, all-to-all
twice is the identity, every All-Reduce output is bit-identical).
"""

from . import bf16, fold, collectives, moe, chain, protocol  # noqa: F401
