"""The decode chain of back-to-back All-Reduces (oracle; test infrastructure only).

SiFAR: Synchronization-Free All-Reduce for Low-Latency LLM Inference (review
page, Fig. 2): a tensor-parallel decode step issues two All-Reduces per layer,
so a 32-layer step is a chain of 64.  Whatever the orchestration -- top and
bottom barriers, dual buffering, or speculative reduction validated by a
reduced flag -- each epoch's result must equal the plain All-Reduce of that
epoch's R payloads (referee report on §8.1: the speculative variant was checked
to match the barrier variant exactly over 100k iterations).  So the oracle of
the chain is the per-epoch All-Reduce, with no orchestration at all.
"""

from . import collectives, fold


def allreduce_chain(ins_by_epoch, dtype="bf16"):
    """ins_by_epoch[e][r] -> list over epochs of the reduced payload.

    Every rank's output at epoch e is this same array (bit-identical).
    """
    return [fold.reduce(list(ins), dtype) for ins in ins_by_epoch]


def collective_chain(name, ins_by_epoch, dtype="bf16", root=None):
    """A chain of any of the seven named collectives: epoch e's outputs are the
    plain collective of that epoch's R inputs (Purlin news page, "The Purlin
    PDF describes a three-layer design": the orchestration layer is reused
    unchanged whatever collective the datapath runs).  Returns, per epoch, the
    list of R outputs (None where the output layout gives a rank nothing).
    ``root`` defaults to the root the seven-collective workload uses."""
    return [collectives.named(name, list(ins), dtype, root=root) for ins in ins_by_epoch]
