"""Torch-facing binding of librrb: plans, Atom copy / reduce, MoE, SNAC chain.

PyTorch supplies device memory and the current stream; every step of the
datapath runs in librrb's HIP kernels.  Tensors are passed by pointer after
the checks below; bf16 data is a torch.bfloat16 tensor or an int16 / uint16
view of bf16 bit patterns, fp32 data a torch.float32 tensor.  Every tensor
must be contiguous, on the current GPU, and hold at least the elements the
plan or chain reads or writes there; anything else raises ValueError before
the library is called (an undersized or strided buffer would otherwise become
an out-of-bounds device access).
"""

import ctypes
import sys

import torch

from . import _lib as L

# Element types each library dtype accepts.
_BF16_TYPES = tuple(t for t in (torch.bfloat16, torch.int16, getattr(torch, "uint16", None))
                    if t is not None)
_F32_TYPES = (torch.float32,)


def _accepts(dtype_code):
    return _BF16_TYPES if dtype_code == L.RRB_BF16 else _F32_TYPES


def _on_gpu(t, what):
    if t.device.type != "cuda" or t.device.index != torch.cuda.current_device():
        raise ValueError(f"{what}: tensor on {t.device}, not on the current GPU")


def _check_tensor(t, what, dtype_code, min_elems):
    """Raise ValueError unless `t` is a contiguous tensor of the library dtype
    with at least `min_elems` elements (the device is checked separately)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype not in _accepts(dtype_code):
        names = "bfloat16, int16 or uint16" if dtype_code == L.RRB_BF16 else "float32"
        raise ValueError(f"{what}: dtype {t.dtype} is not {names}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor is not contiguous")
    if t.numel() < min_elems:
        raise ValueError(f"{what}: {t.numel()} elements, at least {min_elems} needed")


def _check_rank_list(tensors, R, counts, dtype_code, what):
    """Per-rank buffers: at most R entries; entry r is required (and sized)
    when counts[r] > 0 and may be None otherwise.  Returns the tensors given."""
    if tensors is None or len(tensors) > R:
        raise ValueError(f"{what}: expected a list of at most {R} tensors")
    given = []
    for r in range(R):
        t = tensors[r] if r < len(tensors) else None
        if counts[r] > 0 and t is None:
            raise ValueError(f"{what}[{r}]: rank {r} needs a buffer of {counts[r]} elements")
        if t is not None:
            _check_tensor(t, f"{what}[{r}]", dtype_code, counts[r])
            given.append((t, f"{what}[{r}]"))
    return given


def _check_aux(t, what, dtypes, min_elems):
    """An optional auxiliary array (stats, stagger, routing); returns it with
    its name for the device check, or nothing when absent."""
    if t is None:
        return []
    if not isinstance(t, torch.Tensor) or t.dtype not in dtypes:
        raise ValueError(f"{what}: expected a tensor of {' or '.join(map(str, dtypes))}")
    if not t.is_contiguous() or t.numel() < min_elems:
        raise ValueError(f"{what}: expected a contiguous tensor of at least {min_elems} elements")
    return [(t, what)]


def _all_on_gpu(checked):
    for t, what in checked:
        _on_gpu(t, what)


# layout kinds, for collective()
PARTIAL = L.RRB_PARTIAL
REPLICATED = L.RRB_REPLICATED
SHARD = L.RRB_SHARD
BLOCK_ROW = L.RRB_BLOCK_ROW
BLOCK_COL = L.RRB_BLOCK_COL


def ROOT(rho):
    return (L.RRB_ROOT, int(rho))


def _layout(x):
    if isinstance(x, tuple):
        return L.Layout(int(x[0]), int(x[1]))
    return L.Layout(int(x), 0)


def _dtype_code(dtype):
    if dtype in ("bf16", torch.bfloat16, L.RRB_BF16):
        return L.RRB_BF16
    if dtype in ("f32", torch.float32, L.RRB_F32):
        return L.RRB_F32
    raise ValueError(f"unsupported dtype {dtype!r}")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptrs(tensors, R):
    out = []
    for r in range(R):
        t = tensors[r] if r < len(tensors) else None
        out.append(None if t is None else t.data_ptr())
    return L.ptr_array(out)


_OPS = {"copy": L.RRB_COPY, "reduce": L.RRB_REDUCE_SUM, "reduce_tree": L.RRB_REDUCE_SUM_TREE}


def _op_code(op):
    """'copy', 'reduce' (fixed rank order) or 'reduce_tree' (tree order)."""
    if isinstance(op, int):
        return op  # passed through; the library validates it
    if op not in _OPS:
        raise ValueError(f"unknown op {op!r}")
    return _OPS[op]


class Plan:
    """A layout-naming spec compiled to an index map (rrb_plan_create)."""

    def _check(self, status, where):
        return L.check(status, where, self._lib)

    def __init__(self, nranks, count, dtype, in_layout, out_layout, op):
        spec = L.Spec()
        spec.nranks = int(nranks)
        spec.dtype = _dtype_code(dtype)
        spec.count = int(count)
        spec.in_ = _layout(in_layout)
        spec.out = _layout(out_layout)
        spec.op = _op_code(op)
        spec.reserved = 0
        self._lib = L.lib()
        h = ctypes.c_void_p()
        self._check(self._lib.rrb_plan_create(ctypes.byref(spec), ctypes.byref(h)), "rrb_plan_create")
        self.handle = h
        self.nranks = int(nranks)
        self.op = spec.op
        self.dtype = spec.dtype
        self._ws = None
        self._query()

    def _query(self):
        R = self.nranks
        ws = ctypes.c_size_t()
        inc = (ctypes.c_int64 * R)()
        outc = (ctypes.c_int64 * R)()
        self._check(self._lib.rrb_plan_query(self.handle, ctypes.byref(ws), inc, outc), "rrb_plan_query")
        self.workspace_bytes = ws.value
        self.in_count = list(inc)
        self.out_count = list(outc)

    def segments(self):
        n = ctypes.c_int32()
        self._check(self._lib.rrb_plan_segments(self.handle, None, 0, ctypes.byref(n)), "rrb_plan_segments")
        arr = (L.Segment * max(1, n.value))()
        self._check(self._lib.rrb_plan_segments(self.handle, arr, n.value, ctypes.byref(n)),
                "rrb_plan_segments")
        return [(s.src_rank, s.src_off, s.dst_off, s.len, s.dst_mask) for s in arr[:n.value]]

    def bind(self, device=None, stream=None):
        """Allocate (torch) and upload the device-side map if the plan has one."""
        if self.workspace_bytes:
            dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
            self._ws = torch.empty(self.workspace_bytes + 256, dtype=torch.uint8, device=dev)
            base = self._ws.data_ptr()
            aligned = (base + 255) // 256 * 256
            self._check(self._lib.rrb_plan_bind(self.handle, ctypes.c_void_p(aligned),
                                            self.workspace_bytes, _stream(stream)), "rrb_plan_bind")
        return self

    def check_buffers(self, ins, outs):
        """ValueError unless ins / outs fit the plan (see the module doc)."""
        _all_on_gpu(_check_rank_list(ins, self.nranks, self.in_count, self.dtype, "ins") +
                    _check_rank_list(outs, self.nranks, self.out_count, self.dtype, "outs"))

    def run(self, ins, outs, stream=None, weights=None):
        """Atom copy or reduce, whichever the plan names, on torch's stream.
        weights: MoE combine plans only, float32 [tokens, topk] in the
        routing order (replaces the plan's weights for this call)."""
        if weights is not None and getattr(self, "tk", None) is None:
            raise ValueError("weights apply to MoE combine plans only")
        self.check_buffers(ins, outs)
        if self.op == L.RRB_COPY:
            self._check(self._lib.rrb_copy(self.handle, _ptrs(ins, self.nranks), _ptrs(outs, self.nranks),
                                       _stream(stream)), "rrb_copy")
            return
        wp = None
        if weights is not None:
            rows = getattr(self, "tk", None)
            if rows is None:
                raise ValueError("weights apply to MoE combine plans only")
            _all_on_gpu(_check_aux(weights, "weights", _F32_TYPES, rows))
            wp = weights.data_ptr()
        self._check(self._lib.rrb_reduce(self.handle, _ptrs(ins, self.nranks), _ptrs(outs, self.nranks),
                                     wp, _stream(stream)), "rrb_reduce")

    def close(self):
        """Release the library handle now (also done when the object is collected)."""
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self._lib.rrb_plan_destroy(h)
        self.handle = None

    def __del__(self):
        self.close()  # host memory only: safe at interpreter exit


_PLANS = {}


def plan(nranks, count, dtype, in_layout, out_layout, op):
    key = (int(nranks), int(count), _dtype_code(dtype), in_layout, out_layout, op)
    p = _PLANS.get(key)
    if p is None:
        p = Plan(nranks, count, dtype, in_layout, out_layout, op)
        _PLANS[key] = p
    return p


def _dtype_of(t):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype in _BF16_TYPES:
        return L.RRB_BF16
    if t.dtype in _F32_TYPES:
        return L.RRB_F32
    raise ValueError(f"dtype {t.dtype} is neither bf16 (bfloat16 / int16 / uint16 bit patterns) "
                     "nor float32")


def collective(in_layout, out_layout, op, ins, outs, count, stream=None):
    """Any layout-named collective: the plan is cached per (R, n, dtype, naming, op)."""
    t = next(x for x in ins if x is not None)
    p = plan(len(ins), count, _dtype_of(t), in_layout, out_layout, op)
    p.run(ins, outs, stream)
    return outs


class Bound:
    """A collective with its plan, pointer arrays and entry point resolved
    once; calling it issues the launch on torch's current stream with a
    single ctypes call (for launch-bound loops)."""

    __slots__ = ("_fn", "_h", "_in", "_out", "_keep", "_name")

    def __init__(self, p, ins, outs):
        p.check_buffers(ins, outs)
        if p.op == L.RRB_COPY:
            fn = p._lib.rrb_copy
            self._fn = lambda h, i, o, s: fn(h, i, o, s)
            self._name = "rrb_copy"
        else:
            fn = p._lib.rrb_reduce
            self._fn = lambda h, i, o, s: fn(h, i, o, None, s)
            self._name = "rrb_reduce"
        self._h = p.handle
        self._in = _ptrs(ins, p.nranks)
        self._out = _ptrs(outs, p.nranks)
        self._keep = (p, list(ins), list(outs))  # tensors and plan stay alive

    def __call__(self, stream=None):
        st = self._fn(self._h, self._in, self._out,
                      torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream)
        if st:
            L.check(st, self._name, self._keep[0]._lib)

    def kernels(self):
        """The kernel launches this call issues, as the library names them."""
        return launch_info(self._keep[0], self._keep[1], self._keep[2])


def bound(name, ins, outs, root=None, order="fixed"):
    """Pre-bind one of the seven collectives: bound('all_reduce', ins, outs)()
    launches it.  ``order`` applies to the reducing ones ('fixed' or 'tree')."""
    t = next(x for x in ins if x is not None)
    R = len(ins)
    dt = _dtype_of(t)
    n = {"all_gather": t.numel() * R, "gather": t.numel() * R}.get(name, t.numel())
    spec = {
        "all_reduce": (PARTIAL, REPLICATED, "reduce"),
        "reduce_scatter": (PARTIAL, SHARD, "reduce"),
        "all_gather": (SHARD, REPLICATED, "copy"),
        "all_to_all": (BLOCK_ROW, BLOCK_COL, "copy"),
        "broadcast": (ROOT(root if root is not None else 0), REPLICATED, "copy"),
        "reduce": (PARTIAL, ROOT(root if root is not None else 0), "reduce"),
        "gather": (SHARD, ROOT(root if root is not None else 0), "copy"),
    }[name]
    if spec[2] == "reduce":
        spec = (spec[0], spec[1], _reduce_op(order))
    return Bound(plan(R, n, dt, *spec), ins, outs)


# The seven collectives (count = elements of the logical tensor X).
def _reduce_op(order):
    if order not in ("fixed", "tree"):
        raise ValueError(f"unknown reduce order {order!r}")
    return "reduce" if order == "fixed" else "reduce_tree"


def all_reduce(ins, outs, stream=None, order="fixed"):
    """order: 'fixed' (rank order 0..R-1) or 'tree' (pairwise, opt-in)."""
    return collective(PARTIAL, REPLICATED, _reduce_op(order), ins, outs, ins[0].numel(), stream)


def reduce_scatter(ins, outs, stream=None, order="fixed"):
    return collective(PARTIAL, SHARD, _reduce_op(order), ins, outs, ins[0].numel(), stream)


def all_gather(ins, outs, stream=None):
    return collective(SHARD, REPLICATED, "copy", ins, outs, ins[0].numel() * len(ins), stream)


def all_to_all(ins, outs, stream=None):
    return collective(BLOCK_ROW, BLOCK_COL, "copy", ins, outs, ins[0].numel(), stream)


def broadcast(ins, outs, root, stream=None):
    return collective(ROOT(root), REPLICATED, "copy", ins, outs, ins[root].numel(), stream)


def reduce(ins, outs, root, stream=None, order="fixed"):
    return collective(PARTIAL, ROOT(root), _reduce_op(order), ins, outs, ins[0].numel(), stream)


def gather(ins, outs, root, stream=None):
    return collective(SHARD, ROOT(root), "copy", ins, outs, ins[0].numel() * len(ins), stream)


def launch_info(p, ins, outs):
    """The launches rrb_copy / rrb_reduce would issue for plan `p` on these
    buffers, as the library names them (nothing is launched)."""
    buf = ctypes.create_string_buffer(1024)
    p._check(p._lib.rrb_plan_launch_info(p.handle, _ptrs(ins, p.nranks), _ptrs(outs, p.nranks), buf,
                                        len(buf)), "rrb_plan_launch_info")
    return buf.value.decode()


def empty_kernel(stream=None):
    L.check(L.lib().rrb_empty_kernel(_stream(stream)), "rrb_empty_kernel")


# ---- MoE --------------------------------------------------------------------

class MoePlan(Plan):
    """Row-map plan for expert-parallel dispatch (copy) or combine (reduce)."""

    def __init__(self, nranks, hidden, experts, topk_idx, topk_w, direction, device=None):
        import numpy as np
        idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
        w = np.ascontiguousarray(topk_w, dtype=np.float32)
        T, k = idx.shape
        self._lib = L.lib()
        h = ctypes.c_void_p()
        d = L.RRB_MOE_DISPATCH if direction == "dispatch" else L.RRB_MOE_COMBINE
        self._check(self._lib.rrb_plan_create_rows(int(nranks), int(T), int(hidden), int(experts), int(k),
                                               idx.ctypes.data, w.ctypes.data, d, ctypes.byref(h)),
                "rrb_plan_create_rows")
        self.handle = h
        self.nranks = int(nranks)
        self.op = L.RRB_COPY if d == L.RRB_MOE_DISPATCH else L.RRB_REDUCE_SUM
        self.dtype = L.RRB_BF16
        self.hidden = int(hidden)
        self._ws = None
        self._query()
        self.rows_per_rank = [(c if d == L.RRB_MOE_DISPATCH else i) // self.hidden
                              for i, c in zip(self.in_count, self.out_count)]
        self.tk = int(T) * int(k) if d == L.RRB_MOE_COMBINE else None
        self.bind(device)


class MoeDevicePlan(Plan):
    """Row-map plan whose maps are built on the GPU by route() each step.

    The receive side is one arena of tokens*topk rows (rank regions back to
    back); pass it as element 0 of the receive-side tensor list.  A combine
    plan can share the dispatch plan's workspace (share=dispatch_plan), so one
    route() serves both.
    """

    def __init__(self, nranks, tokens, hidden, experts, topk, direction, share=None, device=None):
        self._lib = L.lib()
        h = ctypes.c_void_p()
        d = L.RRB_MOE_DISPATCH if direction == "dispatch" else L.RRB_MOE_COMBINE
        self._check(self._lib.rrb_plan_create_rows_device(int(nranks), int(tokens), int(hidden),
                                                      int(experts), int(topk), d, ctypes.byref(h)),
                "rrb_plan_create_rows_device")
        self.handle = h
        self.nranks = int(nranks)
        self.op = L.RRB_COPY if d == L.RRB_MOE_DISPATCH else L.RRB_REDUCE_SUM
        self.dtype = L.RRB_BF16
        self.tokens, self.hidden, self.experts, self.topk = int(tokens), int(hidden), int(experts), int(topk)
        self.tk = self.tokens * self.topk if d == L.RRB_MOE_COMBINE else None
        self._ws = None
        self._query()
        if share is not None:
            self._ws = share._ws
            base = (self._ws.data_ptr() + 255) // 256 * 256
            self._check(self._lib.rrb_plan_bind(self.handle, ctypes.c_void_p(base), self.workspace_bytes,
                                            _stream()), "rrb_plan_bind")
        else:
            self.bind(device)

    def route(self, topk_idx, topk_w, rank_offsets=None, stream=None):
        """topk_idx int32 [T, k], topk_w float32 [T, k]: device tensors."""
        n = self.tokens * self.topk
        if topk_idx is None or topk_w is None:
            raise ValueError("topk_idx and topk_w are required")
        _all_on_gpu(_check_aux(topk_idx, "topk_idx", (torch.int32,), n) +
                    _check_aux(topk_w, "topk_w", _F32_TYPES, n) +
                    _check_aux(rank_offsets, "rank_offsets", (torch.int32,), self.nranks + 1))
        self._check(self._lib.rrb_moe_route(
            self.handle, ctypes.c_void_p(topk_idx.data_ptr()), ctypes.c_void_p(topk_w.data_ptr()),
            ctypes.c_void_p(rank_offsets.data_ptr() if rank_offsets is not None else 0),
            _stream(stream)), "rrb_moe_route")

    def check(self, stream=None):
        self._check(self._lib.rrb_moe_route_check(self.handle, _stream(stream)), "rrb_moe_route_check")


# ---- SNAC chain -------------------------------------------------------------

VARIANTS = {"barrier": 0, "dual": L.RRB_SNAC_DUAL_BUFFER,
            "speculative": L.RRB_SNAC_DUAL_BUFFER | L.RRB_SNAC_SPECULATIVE,
            "speculative_always": L.RRB_SNAC_DUAL_BUFFER | L.RRB_SNAC_SPECULATIVE | L.RRB_SNAC_SPEC_ALWAYS,
            "graph": L.RRB_SNAC_GRAPH,
            "twoshot": L.RRB_SNAC_TWOSHOT | L.RRB_SNAC_DUAL_BUFFER,
            "lamport": L.RRB_SNAC_LAMPORT | L.RRB_SNAC_DUAL_BUFFER}


class SnacChain:
    """A bound SNAC handle: back-to-back All-Reduces in one persistent kernel."""

    def _check(self, status, where):
        return L.check(status, where, self._lib)

    def __init__(self, nranks, count, dtype="bf16", variant="dual", slices=0, device=None,
                 stream=None, cooperative=False):
        self._lib = L.lib()
        h = ctypes.c_void_p()
        flags = VARIANTS[variant] | (L.RRB_SNAC_COOPERATIVE if cooperative else 0)
        self._check(self._lib.rrb_snac_create(int(nranks), int(count), _dtype_code(dtype),
                                          flags, int(slices), ctypes.byref(h)),
                "rrb_snac_create")
        self.handle = h
        self.nranks = int(nranks)
        self.count = int(count)
        self.variant = variant
        self.dtype = _dtype_code(dtype)
        self.strides = (self.count, self.count)  # elements per rank in d_in / d_out
        ws = ctypes.c_size_t()
        self._check(self._lib.rrb_snac_workspace(h, ctypes.byref(ws)), "rrb_snac_workspace")
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self._ws = torch.empty(ws.value + 256, dtype=torch.uint8, device=dev)
        base = (self._ws.data_ptr() + 255) // 256 * 256
        self._check(self._lib.rrb_snac_bind(h, ctypes.c_void_p(base), ws.value, _stream(stream)),
                "rrb_snac_bind")

    def check_buffers(self, inp, out, stats=None, stagger=None):
        """ValueError unless inp is [epochs, R, in_stride], out is [epochs, R,
        out_stride] (elements), stats an int64[4] and stagger an int32[R]."""
        R = self.nranks
        checked = []
        for t, what, n in ((inp, "inp", self.strides[0]), (out, "out", self.strides[1])):
            if not isinstance(t, torch.Tensor) or t.dim() != 3 or t.shape[1] != R or t.shape[2] != n:
                raise ValueError(f"{what}: expected a tensor of shape [epochs, {R}, {n}]")
            _check_tensor(t, what, self.dtype, 0)
            checked.append((t, what))
        if inp.shape[0] != out.shape[0]:
            raise ValueError("inp and out hold different numbers of epochs")
        checked += _check_aux(stats, "stats", (torch.int64,), 4)
        checked += _check_aux(stagger, "stagger", (torch.int32,), R)
        _all_on_gpu(checked)

    def run(self, inp, out, stats=None, stagger=None, spin_limit=0, stream=None):
        """inp, out: [epochs, R, count] device tensors; stats: int64[4] device tensor."""
        self.check_buffers(inp, out, stats, stagger)
        E = inp.shape[0]
        self._check(self._lib.rrb_snac_allreduce_chain(
            self.handle, int(E), ctypes.c_void_p(inp.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(stats.data_ptr() if stats is not None else 0),
            ctypes.c_void_p(stagger.data_ptr() if stagger is not None else 0),
            int(spin_limit), _stream(stream)), "rrb_snac_allreduce_chain")
        return out

    def bound(self, inp, out, stats=None):
        """The chain call with its arguments marshalled once: calling the
        result runs `inp.shape[0]` epochs on torch's current stream."""
        self.check_buffers(inp, out, stats)
        fn = self._lib.rrb_snac_chain
        args = (self.handle, ctypes.c_int32(int(inp.shape[0])), ctypes.c_void_p(inp.data_ptr()),
                ctypes.c_void_p(out.data_ptr()),
                ctypes.c_void_p(stats.data_ptr() if stats is not None else 0), ctypes.c_void_p(0),
                ctypes.c_uint32(0))
        keep = (inp, out, stats)

        def call():
            st = fn(*args, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st:
                L.check(st, "rrb_snac_chain", self._lib)
        call.keep = keep
        return call

    def check(self, stream=None):
        self._check(self._lib.rrb_snac_check(self.handle, _stream(stream)), "rrb_snac_check")

    def close(self):
        """Destroy the library handle now (a graph-mode handle releases its
        HIP graph here).  Call it before the interpreter exits: collection
        at exit skips the destroy, since the HIP runtime may already be gone."""
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            self._lib.rrb_snac_destroy(h)
        self.handle = None

    def __del__(self):
        if sys.is_finalizing():
            return
        self.close()


def allreduce_chain_noalloc(inp, out, variant="dual", stats=None, spin_limit=0, stream=None,
                            cooperative=False):
    """`inp.shape[0]` chained All-Reduces of inp [epochs, R, count] into out,
    with the library's static per-GPU scratch instead of a workspace
    (rrb_snac_allreduce_chain_noalloc: no device allocation).  variant:
    barrier, dual, speculative, speculative_always or twoshot.  Calls that
    overlap on one GPU race; a wait that ran out shows in stats[2]."""
    if variant not in ("barrier", "dual", "speculative", "speculative_always", "twoshot"):
        raise ValueError(f"variant {variant!r} has no allocation-free form")
    if not isinstance(inp, torch.Tensor) or inp.dim() != 3:
        raise ValueError("inp: expected a tensor of shape [epochs, R, count]")
    E, R, n = inp.shape
    dt = _dtype_of(inp)
    checked = []
    for t, what in ((inp, "inp"), (out, "out")):
        if not isinstance(t, torch.Tensor) or tuple(t.shape) != (E, R, n):
            raise ValueError(f"{what}: expected a tensor of shape [{E}, {R}, {n}]")
        _check_tensor(t, what, dt, 0)
        checked.append((t, what))
    checked += _check_aux(stats, "stats", (torch.int64,), 4)
    _all_on_gpu(checked)
    flags = VARIANTS[variant] | (L.RRB_SNAC_COOPERATIVE if cooperative else 0)
    L.check(L.lib().rrb_snac_allreduce_chain_noalloc(
        int(R), int(n), dt, flags, 0, int(E), ctypes.c_void_p(inp.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(stats.data_ptr() if stats is not None else 0),
        int(spin_limit), _stream(stream)), "rrb_snac_allreduce_chain_noalloc")
    return out


PLAN_CHAIN_VARIANTS = {"barrier": 0, "dual": L.RRB_SNAC_DUAL_BUFFER,
                       "speculative": L.RRB_SNAC_DUAL_BUFFER | L.RRB_SNAC_SPECULATIVE,
                       "graph": L.RRB_SNAC_GRAPH}


class SnacPlanChain(SnacChain):
    """A bound SNAC handle chaining any layout-named collective (a Plan):
    back-to-back collectives of that plan in one persistent kernel (or a
    graph of Atom launches for variant 'graph').  Inputs are
    [epochs, R, in_stride] and outputs [epochs, R, out_stride] in elements
    (``strides``)."""

    def __init__(self, plan, variant="dual", slices=0, device=None, stream=None,
                 cooperative=False):
        self._lib = L.lib()
        h = ctypes.c_void_p()
        flags = PLAN_CHAIN_VARIANTS[variant] | (L.RRB_SNAC_COOPERATIVE if cooperative else 0)
        self._check(self._lib.rrb_snac_create_plan(plan.handle, flags, int(slices), ctypes.byref(h)),
                "rrb_snac_create_plan")
        self.handle = h
        self.nranks = plan.nranks
        self.variant = variant
        self.dtype = plan.dtype
        self.esize = 4 if plan.dtype == L.RRB_F32 else 2
        si, so = ctypes.c_int64(), ctypes.c_int64()
        self._check(self._lib.rrb_snac_strides(h, ctypes.byref(si), ctypes.byref(so)), "rrb_snac_strides")
        self.strides = (si.value // self.esize, so.value // self.esize)
        ws = ctypes.c_size_t()
        self._check(self._lib.rrb_snac_workspace(h, ctypes.byref(ws)), "rrb_snac_workspace")
        dev = device if device is not None else torch.device("cuda", torch.cuda.current_device())
        self._ws = torch.empty(ws.value + 256, dtype=torch.uint8, device=dev)
        base = (self._ws.data_ptr() + 255) // 256 * 256
        self._check(self._lib.rrb_snac_bind(h, ctypes.c_void_p(base), ws.value, _stream(stream)),
                "rrb_snac_bind")

    def run(self, inp, out, stats=None, stagger=None, spin_limit=0, stream=None):
        """inp: [epochs, R, in_stride], out: [epochs, R, out_stride] device tensors."""
        self.check_buffers(inp, out, stats, stagger)
        E = inp.shape[0]
        self._check(self._lib.rrb_snac_chain(
            self.handle, int(E), ctypes.c_void_p(inp.data_ptr()), ctypes.c_void_p(out.data_ptr()),
            ctypes.c_void_p(stats.data_ptr() if stats is not None else 0),
            ctypes.c_void_p(stagger.data_ptr() if stagger is not None else 0),
            int(spin_limit), _stream(stream)), "rrb_snac_chain")
        return out
