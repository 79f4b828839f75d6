"""ctypes declarations of librrb's C ABI (include/rrb.h).  Marshalling only."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librrb.so")
# The same library with the SNAC chains built with memory-model release /
# acquire ordering of their flags (RRB_SNAC_FENCES=1); lib() loads it when the
# environment sets RRB_FENCED=1.
LIB_FENCED_PATH = os.path.join(_HERE, "librrb_fenced.so")

RRB_OK = 0
RRB_EINVAL = -1
RRB_EUNSUPPORTED = -2
RRB_EHIP = -3
RRB_ETIMEOUT = -4
RRB_ENOMEM = -5

RRB_BF16 = 0
RRB_F32 = 1
RRB_COPY = 0
RRB_REDUCE_SUM = 1
RRB_REDUCE_SUM_TREE = 2

RRB_PARTIAL = 0
RRB_REPLICATED = 1
RRB_SHARD = 2
RRB_ROOT = 3
RRB_BLOCK_ROW = 4
RRB_BLOCK_COL = 5

RRB_MOE_DISPATCH = 0
RRB_MOE_COMBINE = 1

RRB_SNAC_DUAL_BUFFER = 1
RRB_SNAC_SPECULATIVE = 2
RRB_SNAC_GRAPH = 4
RRB_SNAC_TWOSHOT = 8
RRB_SNAC_LAMPORT = 16
RRB_SNAC_COOPERATIVE = 32
RRB_SNAC_SPEC_ALWAYS = 64

RRB_MAX_RANKS = 16

# Every symbol include/rrb.h declares.
EXPORTS = (
    "rrb_status_string", "rrb_last_error", "rrb_abi_version",
    "rrb_plan_create", "rrb_plan_create_rows", "rrb_plan_create_rows_device", "rrb_moe_route",
    "rrb_moe_route_check", "rrb_plan_query", "rrb_plan_bind",
    "rrb_plan_segments", "rrb_plan_destroy",
    "rrb_copy", "rrb_reduce", "rrb_plan_launch_info", "rrb_empty_kernel",
    "rrb_snac_create", "rrb_snac_workspace", "rrb_snac_bind", "rrb_snac_allreduce_chain",
    "rrb_snac_create_plan", "rrb_snac_strides", "rrb_snac_chain",
    "rrb_snac_allreduce_chain_noalloc", "rrb_snac_check", "rrb_snac_destroy", "rrb_snac_fenced",
)


class Layout(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("root", ctypes.c_int32)]


class Spec(ctypes.Structure):
    _fields_ = [("nranks", ctypes.c_int32), ("dtype", ctypes.c_int32), ("count", ctypes.c_int64),
                ("in_", Layout), ("out", Layout), ("op", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class Segment(ctypes.Structure):
    _fields_ = [("src_off", ctypes.c_int64), ("dst_off", ctypes.c_int64), ("len", ctypes.c_int64),
                ("src_rank", ctypes.c_int32), ("dst_mask", ctypes.c_uint32)]


class SnacStats(ctypes.Structure):
    _fields_ = [("misspec", ctypes.c_ulonglong), ("retries", ctypes.c_ulonglong),
                ("timeouts", ctypes.c_ulonglong), ("epochs", ctypes.c_ulonglong)]


class RrbError(RuntimeError):
    def __init__(self, status, where, message):
        super().__init__(f"{where}: {message} (status {status})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t

_SIGS = {
    "rrb_status_string": (ctypes.c_char_p, [_I32]),
    "rrb_last_error": (ctypes.c_char_p, []),
    "rrb_abi_version": (_I32, []),
    "rrb_plan_create": (_I32, [ctypes.POINTER(Spec), ctypes.POINTER(_P)]),
    "rrb_plan_create_rows": (_I32, [_I32, _I64, _I64, _I32, _I32, _P, _P, _I32, ctypes.POINTER(_P)]),
    "rrb_plan_create_rows_device": (_I32, [_I32, _I64, _I64, _I32, _I32, _I32, ctypes.POINTER(_P)]),
    "rrb_moe_route": (_I32, [_P, _P, _P, _P, _P]),
    "rrb_moe_route_check": (_I32, [_P, _P]),
    "rrb_plan_query": (_I32, [_P, ctypes.POINTER(_SZ), _P, _P]),
    "rrb_plan_bind": (_I32, [_P, _P, _SZ, _P]),
    "rrb_plan_segments": (_I32, [_P, ctypes.POINTER(Segment), _I32, ctypes.POINTER(_I32)]),
    "rrb_plan_destroy": (None, [_P]),
    "rrb_copy": (_I32, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), _P]),
    "rrb_reduce": (_I32, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), _P, _P]),
    "rrb_plan_launch_info": (_I32, [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.c_char_p, _I32]),
    "rrb_empty_kernel": (_I32, [_P]),
    "rrb_snac_create": (_I32, [_I32, _I64, _I32, _U32, _I32, ctypes.POINTER(_P)]),
    "rrb_snac_workspace": (_I32, [_P, ctypes.POINTER(_SZ)]),
    "rrb_snac_bind": (_I32, [_P, _P, _SZ, _P]),
    "rrb_snac_allreduce_chain": (_I32, [_P, _I32, _P, _P, _P, _P, _U32, _P]),
    "rrb_snac_create_plan": (_I32, [_P, _U32, _I32, ctypes.POINTER(_P)]),
    "rrb_snac_strides": (_I32, [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "rrb_snac_chain": (_I32, [_P, _I32, _P, _P, _P, _P, _U32, _P]),
    "rrb_snac_allreduce_chain_noalloc": (_I32, [_I32, _I64, _I32, _U32, _I32, _I32, _P, _P, _P, _U32, _P]),
    "rrb_snac_check": (_I32, [_P, _P]),
    "rrb_snac_destroy": (None, [_P]),
    "rrb_snac_fenced": (_I32, []),
}
_loaded = {}


def _open(path):
    if path not in _loaded:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{os.path.basename(path)} is not built at {path}; run "
                "`python -m reduce_rank_buffers_amd.build` (there is no fallback path)")
        l = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _loaded[path] = l
    return _loaded[path]


def lib():
    """The loaded librrb (librrb_fenced.so if RRB_FENCED=1); raises loudly if
    it was never built."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_FENCED_PATH if os.environ.get("RRB_FENCED") == "1" else LIB_PATH)
    return _lib


def select(fenced):
    """Make lib() return the fenced-ordering build (True) or the default one
    (False) from now on, for objects created afterwards; returns the library
    it replaced (None if none was loaded).  Objects keep the library they
    were created with."""
    global _lib
    prev = _lib
    _lib = _open(LIB_FENCED_PATH if fenced else LIB_PATH)
    return prev


def restore(prev):
    """Undo select(): lib() returns `prev` again (or loads afresh if None)."""
    global _lib
    _lib = prev


def check(status, where, l=None):
    """Raise RrbError for a failed call; `l` is the library the call went to
    (default: lib()), whose thread-local last error holds the message."""
    if status != RRB_OK:
        l = lib() if l is None else l
        msg = l.rrb_last_error().decode() or l.rrb_status_string(status).decode()
        raise RrbError(status, where, msg)
    return status


def ptr_array(ptrs):
    arr = (_P * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr
