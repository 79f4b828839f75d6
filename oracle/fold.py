"""The Atom reduce primitive, fixed rank order (oracle; test infrastructure only).

Purlin: Separating Orchestration from the Datapath of Collectives, "The Purlin
PDF describes a three-layer design": the datapath below the orchestration layer
offers two primitives, copy and reduce.  Reduce combines the same element of
several rank payloads.  The decode workload states the arithmetic: accumulate
in fp32 in fixed rank order 0..R-1, then round once to bf16 with
round-to-nearest-even.

Definition written out (one IEEE binary32 addition per step, numpy float32
arithmetic is correctly rounded):

    s_0     = f32(x_0[j])
    s_r     = fl32(s_{r-1} + f32(x_r[j]))      r = 1 .. R-1
    result  = RNE_bf16(s_{R-1})                 (or s_{R-1} for fp32 data)

The fold starts from x_0 rather than from +0.0 (a reading: the two differ only
when every term is -0, where starting at x_0 keeps -0).

Parity pinned by: an exact rational emulation of binary32 addition on tiny
inputs (tests/test_oracle_fold.py), closed forms and the recursive-summation
error bound.

Tree order (an optional, flagged variant; a reading -- the pages fix no tree).
Pairwise summation level by level: adjacent items (0, 1), (2, 3), ... are
added with one binary32 addition each, an odd last item passes up unchanged,
until one item is left; for R = 8 that is
((x0 + x1) + (x2 + x3)) + ((x4 + x5) + (x6 + x7)).  For R <= 3 it coincides
with the fixed order.  Its result may differ from the fixed-order fold by
rounding; the bound it must meet against that fold is
|d| <= max(1 ulp_bf16(y), 2 (R - 1) 2^-24 sum |x_r|).  Pinned by hand-worked
cases where the association changes the result, the exact emulation of the
same tree, and that bound.
"""

import numpy as np

from . import bf16


def fold_f32(xs):
    """Fixed-order fp32 sum of R float32 arrays (list or [R, ...] array)."""
    xs = [np.asarray(x, dtype=np.float32) for x in xs]
    if not xs:
        raise ValueError("fold needs at least one rank")
    s = xs[0].copy()
    with np.errstate(over="ignore", invalid="ignore"):  # IEEE inf / NaN results
        for x in xs[1:]:
            s = (s + x).astype(np.float32)
    return s


def reduce_bf16(ins):
    """R bf16 payloads (uint16 arrays of equal shape) -> bf16 fixed-order sum."""
    return bf16.rne(fold_f32([bf16.widen(x) for x in ins]))


def reduce_f32(ins):
    """R float32 payloads -> float32 fixed-order sum (no final rounding)."""
    return fold_f32(ins)


def fold_tree_f32(xs):
    """Tree-order fp32 sum of R float32 arrays (see the module docstring)."""
    items = [np.asarray(x, dtype=np.float32) for x in xs]
    if not items:
        raise ValueError("fold needs at least one rank")
    with np.errstate(over="ignore", invalid="ignore"):
        while len(items) > 1:
            nxt = [(items[i] + items[i + 1]).astype(np.float32)
                   for i in range(0, len(items) - 1, 2)]
            if len(items) % 2:
                nxt.append(items[-1])
            items = nxt
    return items[0].copy()


def reduce_tree(ins, dtype):
    """Tree-order reduce: bf16 payloads round once at the end, f32 do not."""
    if dtype == "bf16":
        return bf16.rne(fold_tree_f32([bf16.widen(x) for x in ins]))
    if dtype == "f32":
        return fold_tree_f32(ins)
    raise ValueError(f"unknown dtype {dtype!r}")


def reduce(ins, dtype):
    """Dispatch on element type: 'bf16' (uint16 patterns) or 'f32'."""
    if dtype == "bf16":
        return reduce_bf16(ins)
    if dtype == "f32":
        return reduce_f32(ins)
    raise ValueError(f"unknown dtype {dtype!r}")
