"""Seeded synthetic inputs shared by the tests, the bench and the oracle's callers.

This module holds none of the collective datapath's arithmetic: it draws
random numbers and converts them to bf16 with torch's CPU conversion (a
library round-to-nearest-even).  Both the HIP path and the CPU oracle receive
exactly the bits made here, as numpy arrays.

Seeds follow ``numpy.random.default_rng([workload, kind, epoch, rank])`` so
every buffer of every workload can be regenerated independently.

Workloads (sizes are what they are named for, not tuning knobs):

* decode All-Reduce: R = 8 ranks x 4096 bf16, N(0, 1);
* bandwidth sweep: R = 8 ranks x S MiB per rank, S in {1, 4, 16, 64, 256},
  bf16 N(0, 1), plus fp32 N(0, 1) at 64 MiB;
* seven layout-named collectives: R = 8, 16 MiB per rank, bf16 N(0, 1);
* decode chain: payload b x h bf16, b in {1..64}, h in {4096, 8192},
  N(0, 0.02) (sigma 0.02), 64 epochs, fresh data per (epoch, rank);
* MoE: 4096 tokens x 7168 bf16 N(0, 1), logits N(0, 1) [4096, 256],
  softmax then top-8 (the gate; not part of the datapath);
* buffers past 2 GiB (the size-limit tests): drawn on the device by torch's
  seeded generator (``device_normal_bf16``), since a host draw of that size
  is slow; the oracle checks sampled elements copied back from these inputs.
"""

import numpy as np
import torch

WL_DECODE = 1
WL_SWEEP = 2
WL_SEVEN = 3
WL_CHAIN = 4
WL_MOE = 5


def rng(workload, kind=0, epoch=0, rank=0):
    return np.random.default_rng([int(workload), int(kind), int(epoch), int(rank)])


def to_bf16_bits(x_f32):
    """float32 numpy array -> bf16 bit patterns (uint16) via torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_f32(n, sigma=1.0, *key):
    x = rng(*key).standard_normal(int(n), dtype=np.float32)
    if sigma != 1.0:
        x = (x * np.float32(sigma)).astype(np.float32)
    return x


def normal_bf16(n, sigma=1.0, *key):
    """n bf16 values ~ N(0, sigma^2): sample fp32, scale in fp32, round to bf16."""
    return to_bf16_bits(normal_f32(n, sigma, *key))


def rank_payloads(n, R=8, dtype="bf16", sigma=1.0, workload=WL_SWEEP, kind=0, epoch=0):
    """R independent payloads of n elements: uint16 (bf16 bits) or float32."""
    if dtype == "bf16":
        return [normal_bf16(n, sigma, workload, kind, epoch, r) for r in range(R)]
    if dtype == "f32":
        return [normal_f32(n, sigma, workload, kind, epoch, r) for r in range(R)]
    raise ValueError(dtype)


def decode_allreduce(R=8, n=4096):
    """Decode All-Reduce inputs: R x 4096 bf16 N(0,1)."""
    return rank_payloads(n, R, "bf16", 1.0, WL_DECODE, 0, 0)


def sweep(S_mib, R=8, dtype="bf16"):
    """Bandwidth sweep inputs: S MiB per rank (the full logical tensor)."""
    esz = 2 if dtype == "bf16" else 4
    n = (int(S_mib) << 20) // esz
    kind = int(S_mib) if dtype == "bf16" else 1000 + int(S_mib)
    return rank_payloads(n, R, dtype, 1.0, WL_SWEEP, kind, 0)


def chain(epochs, R, n, sigma=0.02, kind=None):
    """Decode-chain inputs: array [epochs, R, n] of bf16 bits, N(0, sigma^2)."""
    kind = n if kind is None else kind
    out = np.empty((epochs, R, n), dtype=np.uint16)
    for e in range(epochs):
        for r in range(R):
            out[e, r] = normal_bf16(n, sigma, WL_CHAIN, kind, e, r)
    return out


def moe_routing(T=4096, E=256, k=8, seed_kind=1):
    """The gate: logits N(0,1) [T, E] fp32 -> softmax (float64, cast to fp32)
    -> top-k by descending probability, ties to the lower expert id.

    Weights are the selected probabilities, not renormalised.  Returns
    (idx int32 [T, k], w float32 [T, k]).
    """
    logits = rng(WL_MOE, seed_kind).standard_normal((T, E), dtype=np.float32)
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    idx = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return idx, w


def moe_tokens(T=4096, h=7168, R=8):
    """Token rows [T, h] bf16 N(0,1), split into R source shards of T/R rows."""
    x = normal_bf16(T * h, 1.0, WL_MOE, 0, 0, 0).reshape(T, h)
    tr = T // R
    return [x[r * tr:(r + 1) * tr].copy() for r in range(R)]


def moe_expert_outputs(rows_per_rank, h=7168):
    """Independently seeded stand-in expert outputs in the dispatch layout."""
    return [normal_bf16(int(n) * h, 1.0, WL_MOE, 2, 0, r).reshape(int(n), h)
            for r, n in enumerate(rows_per_rank)]


WL_LARGE = 6


def device_normal_bf16(n, rank, device, kind=0):
    """n bf16 N(0, 1) values drawn on `device` by torch's generator seeded with
    (WL_LARGE, kind, rank): an int16 tensor holding the bf16 bit patterns."""
    g = torch.Generator(device=device)
    g.manual_seed(WL_LARGE * 1_000_003 + int(kind) * 1009 + int(rank))
    x = torch.randn(int(n), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16).view(torch.int16)
