"""Collectives as layout naming + copy | reduce (oracle; test infrastructure only).

Purlin: Separating Orchestration from the Datapath of Collectives, "The Purlin
PDF describes a three-layer design": the top layer specifies a collective as a
naming of an input layout and an output layout plus either a copy or a
reduction.  Nothing else is said about the naming, so this module takes the
plainest reading:

* A logical tensor X of ``n`` elements is what the collective is about.  With
  R ranks it splits into R equal contiguous blocks of ``c = n / R`` elements
  (only layouts that name blocks need ``n % R == 0``).
* A layout says, for every rank, which logical element each of its local
  elements *names*:

  ``PARTIAL``     rank q holds a full-length partial P_q of X (X = sum of P_q).
  ``REPLICATED``  every rank holds all of X.
  ``SHARD``       rank q holds block q of X.
  ``ROOT(rho)``   rank rho holds all of X; other ranks hold nothing.
  ``BLOCK_ROW``   X is an R x R matrix of blocks M[r][q]; rank r holds row r
                  (local block q is M[r][q]).
  ``BLOCK_COL``   rank q holds column q (local block r is M[r][q]).

* ``copy``: every output element receives the input element carrying the same
  name (if several ranks hold it, the lowest rank's copy -- by the layout's
  meaning all copies are equal).
* ``reduce``: the input must be ``PARTIAL``; the output element named X[j]
  receives the fixed-order fold over ranks 0..R-1 of P_r[j] (``fold.py``).
  ``reduce_tree`` is the same with the tree-order fold.

``collective`` below applies that definition element by element (slow; for
small cases).  The seven named collectives are then written out directly from
their plain definitions, each citing where the pages use it; tests check both
agree, which pins the naming reading against the textbook definitions.
"""

import numpy as np

from . import fold

PARTIAL = "PARTIAL"
REPLICATED = "REPLICATED"
SHARD = "SHARD"
BLOCK_ROW = "BLOCK_ROW"
BLOCK_COL = "BLOCK_COL"


def ROOT(rho):
    return ("ROOT", int(rho))


def _kind(layout):
    return layout[0] if isinstance(layout, tuple) else layout


def names(layout, q, R, n):
    """Names of rank q's local elements, in local order, under ``layout``."""
    kind = _kind(layout)
    if kind == PARTIAL:
        return [("P", q, j) for j in range(n)]
    if kind == REPLICATED:
        return [("X", j) for j in range(n)]
    if kind == "ROOT":
        return [("X", j) for j in range(n)] if q == layout[1] else []
    if n % R:
        raise ValueError(f"layout {kind} needs n divisible by R")
    c = n // R
    if kind == SHARD:
        return [("X", q * c + j) for j in range(c)]
    if kind == BLOCK_ROW:
        return [("M", q, j // c, j % c) for j in range(n)]
    if kind == BLOCK_COL:
        return [("M", j // c, q, j % c) for j in range(n)]
    raise ValueError(f"unknown layout {layout!r}")


def collective(in_layout, out_layout, op, ins, R, n, dtype="bf16"):
    """Apply a layout-named collective element by element.

    ``ins[r]`` is rank r's input buffer (or None where the input layout gives
    rank r nothing).  Returns a list of R output buffers; a rank the output
    layout gives nothing to gets None (its buffer is not written).
    """
    in_names = [names(in_layout, r, R, n) for r in range(R)]
    out_names = [names(out_layout, q, R, n) for q in range(R)]
    outs = []
    if op == "copy":
        where = {}
        for r in range(R):
            for i, nm in enumerate(in_names[r]):
                where.setdefault(nm, (r, i))  # lowest rank first
        for q in range(R):
            if not out_names[q]:
                outs.append(None)
                continue
            dt = next(np.asarray(x).dtype for x in ins if x is not None)
            o = np.empty(len(out_names[q]), dtype=dt)
            for i, nm in enumerate(out_names[q]):
                if nm not in where:
                    raise ValueError(f"output name {nm} not held by the input layout")
                r, k = where[nm]
                o[i] = ins[r][k]
            outs.append(o)
        return outs
    if op in ("reduce", "reduce_tree"):
        if _kind(in_layout) != PARTIAL:
            raise ValueError("reduce needs a PARTIAL input layout")
        for q in range(R):
            if not out_names[q]:
                outs.append(None)
                continue
            idx = []
            for nm in out_names[q]:
                if nm[0] != "X":
                    raise ValueError("reduce output must name elements of X")
                idx.append(nm[1])
            idx = np.asarray(idx, dtype=np.int64)
            cols = [np.asarray(ins[r])[idx] for r in range(R)]
            outs.append(fold.reduce(cols, dtype) if op == "reduce" else fold.reduce_tree(cols, dtype))
        return outs
    raise ValueError(f"unknown op {op!r}")


# --- the seven collectives, written from their plain definitions -----------

def all_reduce(ins, dtype="bf16"):
    """Every rank receives the reduction of all R payloads (SiFAR review,
    abstract and Fig. 5: each GPU ends with the full reduced payload)."""
    y = fold.reduce(ins, dtype)
    return [y.copy() for _ in ins]


def reduce_scatter(ins, dtype="bf16"):
    """Rank q receives contiguous chunk q of the reduction (SiFAR review,
    Fig. 6 and Fig. 9: twoshot's first step, each GPU reduces a portion)."""
    R = len(ins)
    n = len(ins[0])
    c = n // R
    return [fold.reduce([x[q * c:(q + 1) * c] for x in ins], dtype) for q in range(R)]


def reduce_root(ins, root, dtype="bf16"):
    """Only rank ``root`` receives the reduction; other outputs untouched."""
    out = [None] * len(ins)
    out[root] = fold.reduce(ins, dtype)
    return out


def all_gather(ins):
    """Every rank receives the concatenation of all R shards in rank order
    (twoshot's second step, SiFAR review abstract and Fig. 6)."""
    y = np.concatenate([np.asarray(x) for x in ins])
    return [y.copy() for _ in ins]


def gather(ins, root):
    """Only rank ``root`` receives the concatenation of all R shards."""
    out = [None] * len(ins)
    out[root] = np.concatenate([np.asarray(x) for x in ins])
    return out


def broadcast(ins, root):
    """Every rank, the root included, receives the root's buffer."""
    return [np.asarray(ins[root]).copy() for _ in ins]


def all_to_all(ins):
    """8x8 block transpose: out_q block r = in_r block q."""
    R = len(ins)
    n = len(ins[0])
    c = n // R
    return [np.concatenate([np.asarray(ins[r])[q * c:(q + 1) * c] for r in range(R)])
            for q in range(R)]


# name -> (input layout, output layout, op) for the seven collectives
SEVEN = {
    "all_reduce": (PARTIAL, REPLICATED, "reduce"),
    "reduce_scatter": (PARTIAL, SHARD, "reduce"),
    "all_gather": (SHARD, REPLICATED, "copy"),
    "all_to_all": (BLOCK_ROW, BLOCK_COL, "copy"),
    "broadcast": (ROOT(3), REPLICATED, "copy"),
    "reduce": (PARTIAL, ROOT(0), "reduce"),
    "gather": (SHARD, ROOT(5), "copy"),
}


def named(name, ins, dtype="bf16", root=None):
    """Run one of the seven by its closed form."""
    if name == "all_reduce":
        return all_reduce(ins, dtype)
    if name == "reduce_scatter":
        return reduce_scatter(ins, dtype)
    if name == "all_gather":
        return all_gather(ins)
    if name == "all_to_all":
        return all_to_all(ins)
    if name == "broadcast":
        return broadcast(ins, 3 if root is None else root)
    if name == "reduce":
        return reduce_root(ins, 0 if root is None else root, dtype)
    if name == "gather":
        return gather(ins, 5 if root is None else root)
    raise ValueError(name)
