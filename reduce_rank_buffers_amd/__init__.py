"""reduce_rank_buffers_amd: an MI355X-native collective datapath on one GPU.

The R ranks are R buffers in one GPU's HBM.  Collectives are named by an input
layout, an output layout and copy | reduce; the HIP library ``librrb.so``
turns the naming into an index map and runs the Atom copy / reduce kernels,
the stage / notify / consume chain and the MoE row maps.  This package is the
argument-marshalling layer over that C ABI; it computes nothing itself, and
it has no fallback: without ``librrb.so`` every call raises.
"""

from .api import (  # noqa: F401
    PARTIAL, REPLICATED, SHARD, BLOCK_ROW, BLOCK_COL, ROOT,
    Plan, MoePlan, MoeDevicePlan, SnacChain, SnacPlanChain, plan, collective,
    all_reduce, reduce_scatter, all_gather, all_to_all, broadcast, reduce, gather,
    empty_kernel, bound, Bound,
)
from ._lib import RrbError, lib  # noqa: F401
