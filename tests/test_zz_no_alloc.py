"""The allocation-free All-Reduce chain (rrb_snac_allreduce_chain_noalloc),
called through the C ABI, against the chain entry point that runs on caller
workspace (rrb_snac_allreduce_chain): bit-exact on two calls in a row, the
second with a smaller input (the shared static scratch keeps the first
call's contents), for every flag protocol; also against the oracle.  The
size limit and the unsupported variants are rejected before any GPU work
(checked on the CPU)."""

import ctypes
import sys

import numpy as np
import pytest
import torch

from oracle import chain as OC
from reduce_rank_buffers_amd import _lib as L, api, inputs

R = 8
FLAGS = {"barrier": 0, "dual": L.RRB_SNAC_DUAL_BUFFER,
         "speculative": L.RRB_SNAC_DUAL_BUFFER | L.RRB_SNAC_SPECULATIVE,
         "twoshot": L.RRB_SNAC_TWOSHOT | L.RRB_SNAC_DUAL_BUFFER}


def test_noalloc_rejects_oversize_and_other_variants(librrb):
    # 8 ranks x 2 MiB: 32 MiB of staging, beyond the 20 MiB array
    st = librrb.rrb_snac_allreduce_chain_noalloc(8, 1 << 20, L.RRB_BF16, L.RRB_SNAC_DUAL_BUFFER, 0, 4,
                                                 None, None, None, 0, None)
    assert st == L.RRB_EUNSUPPORTED
    assert b"static scratch holds" in librrb.rrb_last_error()
    for f in (L.RRB_SNAC_GRAPH, L.RRB_SNAC_LAMPORT | L.RRB_SNAC_DUAL_BUFFER):
        st = librrb.rrb_snac_allreduce_chain_noalloc(8, 4096, L.RRB_BF16, f, 0, 4, None, None, None, 0, None)
        assert st == L.RRB_EUNSUPPORTED
    # 8 ranks x 1 MiB with twoshot (the largest layout) fits: it fails only
    # on the NULL payload, after the size check
    st = librrb.rrb_snac_allreduce_chain_noalloc(8, 1 << 19, L.RRB_BF16, FLAGS["twoshot"], 0, 4,
                                                 None, None, None, 0, None)
    assert st == L.RRB_EINVAL


@pytest.mark.gpu
@pytest.mark.parametrize("variant", list(FLAGS))
def test_noalloc_matches_workspace_chain(variant):
    lib = L.lib()
    dev = torch.device("cuda", 0)
    for call, (E, n) in enumerate([(16, 32768), (8, 4096)]):  # the second call is smaller
        print(f"noalloc {variant} call {call}: {E} epochs x {R} x {n}", file=sys.stderr, flush=True)
        ins_np = inputs.chain(E, R, n, kind=300 + call)
        inp = torch.from_numpy(ins_np.view(np.int16)).to(dev)
        out = torch.full_like(inp, -21555)
        stats = torch.zeros(4, dtype=torch.int64, device=dev)
        api.allreduce_chain_noalloc(inp, out, variant, stats=stats)
        ch = api.SnacChain(R, n, "bf16", variant)
        ref = torch.empty_like(inp)
        ch.run(inp, ref)
        ch.check()
        torch.cuda.synchronize()
        ch.close()
        assert stats[2].item() == 0, f"{variant} call {call}: a wait timed out"
        assert torch.equal(out, ref), f"{variant} call {call}: differs from the workspace chain"
        got = out.cpu().numpy().view(np.uint16)
        for e, w in enumerate(OC.allreduce_chain(ins_np)):
            for r in range(R):
                assert np.array_equal(got[e, r], w), f"{variant} call {call} epoch {e} rank {r}"
