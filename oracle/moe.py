"""Expert-parallel dispatch and combine over R simulated ranks (oracle; test
infrastructure only).

The pages name no MoE datapath of their own (the SiFAR review only evaluates a
large MoE model end to end and cites DeepEP); the MoE workload is an
all-to-all style pair of collectives expressed with the two Atom primitives of
Purlin: Separating Orchestration from the Datapath of Collectives ("The Purlin
PDF describes a three-layer design"): a *copy* by an expert index map
(dispatch) and a *reduce* with weights in fixed expert order (combine).
Readings taken here, since nothing fixes them:

* Expert e lives on rank ``e // (E / R)``.
* Tokens are sharded over the R source ranks, ``T / R`` consecutive tokens per
  rank; global token t is row ``t % (T/R)`` of source rank ``t // (T/R)``.
* Rank r's receive buffer is expert-major over its experts in ascending id,
  and tokens ascend within an expert; no capacity limit, no dropped tokens,
  one copy per (token, expert) pair.
* Combine folds a token's k weighted expert rows in ascending *expert id*
  (not top-k rank order), one binary32 multiply then one binary32 add per
  step (no fused multiply-add), then rounds once to bf16:

      a_1 = fl32(w_1 * f32(z_1)),  a_i = fl32(a_{i-1} + fl32(w_i * f32(z_i))),
      y   = RNE_bf16(a_k).

Parity pinned by: the count/offset invariants, gathering dispatched rows back
reproduces x, one-hot weights give the combine exactly bf16(z) of one slot,
and an exact rational emulation on tiny T and h (tests/test_oracle_moe.py).
"""

import numpy as np

from . import bf16


def expert_tokens(idx, E):
    """For each expert e, the ascending list of tokens routed to it."""
    idx = np.asarray(idx)
    T, k = idx.shape
    lists = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            lists[int(idx[t, j])].append(t)
    return [sorted(l) for l in lists]


def layout(idx, E, R):
    """counts[e], offsets[e] (within its rank's buffer), rows per rank."""
    toks = expert_tokens(idx, E)
    per = E // R
    counts = np.array([len(l) for l in toks], dtype=np.int64)
    offsets = np.zeros(E, dtype=np.int64)
    rows = np.zeros(R, dtype=np.int64)
    for e in range(E):
        r = e // per
        offsets[e] = rows[r]
        rows[r] += counts[e]
    return toks, counts, offsets, rows


def dispatch(x_shards, idx, E):
    """x_shards: R arrays [T/R, h] (any dtype, copied as bits).

    Returns R receive buffers; rank r's buffer is [rows_r, h].
    """
    R = len(x_shards)
    x = np.concatenate([np.asarray(s) for s in x_shards], axis=0)
    h = x.shape[1]
    toks, counts, offsets, rows = layout(idx, E, R)
    per = E // R
    recv = [np.empty((int(rows[r]), h), dtype=x.dtype) for r in range(R)]
    for e in range(E):
        r = e // per
        for i, t in enumerate(toks[e]):
            recv[r][offsets[e] + i] = x[t]
    return recv


def combine(z, idx, w, E, tokens_per_rank):
    """z: R expert-output buffers in the dispatch layout (bf16 patterns).

    idx, w: [T, k] routing; returns R output shards [T/R, h] of bf16.
    """
    R = len(z)
    idx = np.asarray(idx)
    w = np.asarray(w, dtype=np.float32)
    T, k = idx.shape
    h = np.asarray(z[0]).shape[1]
    toks, counts, offsets, rows = layout(idx, E, R)
    per = E // R
    # position of token t within expert e's token list
    pos = [dict((t, i) for i, t in enumerate(toks[e])) for e in range(E)]
    y = np.empty((T, h), dtype=np.uint16)
    for t in range(T):
        order = np.argsort(idx[t], kind="stable")  # ascending expert id
        acc = None
        for j in order:
            e = int(idx[t, j])
            r = e // per
            row = bf16.widen(z[r][offsets[e] + pos[e][t]])
            term = (np.float32(w[t, j]) * row).astype(np.float32)
            acc = term if acc is None else (acc + term).astype(np.float32)
        y[t] = bf16.rne(acc)
    return [y[r * tokens_per_rank:(r + 1) * tokens_per_rank] for r in range(R)]
