"""reduce_rank_buffers_amd: an MI355X-native collective datapath on one GPU.

The R ranks are R buffers in one GPU's HBM.  Collectives are named by an input
layout, an output layout and copy | reduce; the HIP library ``librrb.so``
turns the naming into an index map and runs the Atom copy / reduce kernels,
the stage / notify / consume chain and the MoE row maps.  This package is the
argument-marshalling layer over that C ABI; it computes nothing itself.
"""

__all__ = ["inputs"]
