"""ctypes binding of libfa.so: one Python function per C entry point.

Argument marshalling only. Pointers are passed as Python ints (device
addresses, e.g. ``tensor.data_ptr()``), the stream as an int
(``torch.cuda.current_stream().cuda_stream``). Each function returns the
C status code; :func:`check` turns a nonzero code into :class:`FaError`.
The library must be built (``python -m exact_io_aware_69_amd.build``);
loading fails loudly otherwise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

from . import _srcid

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_u32 = ctypes.c_uint32
_u64 = ctypes.c_uint64

# name -> (restype, argtypes); mirrors include/fa.h
SIGNATURES = {
    "fa_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p]),
    "fa_fwd_blocksparse": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p]),
    "fa_fwd_tiles": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _i, _i, _p]),
    "fa_std_workspace_size": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fa_std_fwd": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _sz, _p]),
    "fa_fa1_workspace_size": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fa_fwd_fa1": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _i, _p, _sz, _p]),
    "fa_bwd_workspace_size": (_i, [_i, _i, _i, _i, ctypes.POINTER(_sz)]),
    "fa_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _sz, _p]),
    "fa_bwd_blocksparse": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _sz, _p]),
    "fa_bwd_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p]),
    "fa_bwd_stage": (_i, [_i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _sz, _p]),
    "fa_fwd_dropout": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _f, _u64, _u32, _p]),
    "fa_bwd_dropout": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _f, _u64, _u32, _p, _sz,
                            _p]),
    "fa_dropout_keep": (_i, [_i, _i, _i, _f, _u64, _u32, _p, _p]),
    "fa_tile_config": (_i, [_i, _i, _i, ctypes.POINTER(_i), ctypes.POINTER(_i)]),
    "fa_fwd_debug_visits": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _p]),
    "fa_bwd_debug_visits": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _sz,
                                 _p, _p, _p]),
    "fa_status_str": (ctypes.c_char_p, [_i]),
    "fa_build_id": (ctypes.c_char_p, []),
    "fa_atomic_add_probe": (_i, [_p, _sz, _i, _i, _p]),
}

FA_OK = 0
STATUS = {
    0: "FA_OK", -1: "FA_ERR_NULL", -2: "FA_ERR_SHAPE", -3: "FA_ERR_UNSUPPORTED_D", -4: "FA_ERR_SCALE",
    -5: "FA_ERR_WORKSPACE", -6: "FA_ERR_MASK", -7: "FA_ERR_HIP", -8: "FA_ERR_ALIGN", -9: "FA_ERR_DROPOUT",
}


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_str(status)} ({status})")


_lib = None


class StaleLibraryError(ImportError):
    """libfa.so was built from sources other than the ones beside it."""


def lib():
    """Load libfa.so once. Raises ImportError if it has not been built, and
    StaleLibraryError if it was built from other sources than the ones in
    this tree (rebuild with `python -m exact_io_aware_69_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with `python -m exact_io_aware_69_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        built = l.fa_build_id().decode()
        want = _srcid.source_id()
        if built != want:
            raise StaleLibraryError(
                f"{LIB_PATH} was built from sources {built}, the tree holds {want}: rebuild with "
                "`python -m exact_io_aware_69_amd.build`")
        _lib = l
    return _lib


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)


def fa_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, stream):
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, int(causal), scale, stream)


def fa_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, stream):
    return lib().fa_fwd_blocksparse(q, k, v, o, lse, B, H, N, d, int(causal), scale, block_mask, stream)


def fa_fwd_tiles(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, bm, bn, stream):
    return lib().fa_fwd_tiles(q, k, v, o, lse, B, H, N, d, int(causal), scale, block_mask, bm, bn, stream)


def fa_std_workspace_size(B, H, N, d):
    """Returns (status, bytes)."""
    out = _sz(0)
    st = lib().fa_std_workspace_size(B, H, N, d, ctypes.byref(out))
    return st, out.value


def fa_std_fwd(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, workspace, workspace_bytes, stream):
    return lib().fa_std_fwd(q, k, v, o, lse, B, H, N, d, int(causal), scale, block_mask, workspace,
                            workspace_bytes, stream)


def fa_fa1_workspace_size(B, H, N, d):
    """Returns (status, bytes)."""
    out = _sz(0)
    st = lib().fa_fa1_workspace_size(B, H, N, d, ctypes.byref(out))
    return st, out.value


def fa_fwd_fa1(q, k, v, o, lse, B, H, N, d, causal, scale, seq_groups, workspace, workspace_bytes, stream):
    return lib().fa_fwd_fa1(q, k, v, o, lse, B, H, N, d, int(causal), scale, seq_groups, workspace, workspace_bytes,
                            stream)


def fa_bwd_workspace_size(B, H, N, d):
    """Returns (status, bytes)."""
    out = _sz(0)
    st = lib().fa_bwd_workspace_size(B, H, N, d, ctypes.byref(out))
    return st, out.value


def fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, workspace, workspace_bytes, stream):
    return lib().fa_bwd(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, int(causal), scale, workspace,
                        workspace_bytes, stream)


def fa_bwd_blocksparse(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, workspace,
                       workspace_bytes, stream):
    return lib().fa_bwd_blocksparse(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, int(causal), scale,
                                    block_mask, workspace, workspace_bytes, stream)


def fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, stream):
    return lib().fa_bwd_noalloc(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, int(causal), scale, block_mask, stream)


def fa_bwd_stage(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, workspace,
                 workspace_bytes, stream):
    return lib().fa_bwd_stage(stage, q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, int(causal), scale, block_mask,
                              workspace, workspace_bytes, stream)


def fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, dropout_p, seed, offset, stream):
    return lib().fa_fwd_dropout(q, k, v, o, lse, B, H, N, d, int(causal), scale, block_mask, dropout_p, seed, offset,
                                stream)


def fa_bwd_dropout(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, dropout_p, seed, offset,
                   workspace, workspace_bytes, stream):
    return lib().fa_bwd_dropout(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, int(causal), scale, block_mask,
                                dropout_p, seed, offset, workspace, workspace_bytes, stream)


def fa_dropout_keep(B, H, N, dropout_p, seed, offset, keep, stream):
    return lib().fa_dropout_keep(B, H, N, dropout_p, seed, offset, keep, stream)


def fa_tile_config(pass_, d, causal):
    """Returns (status, bm, bn)."""
    bm, bn = _i(0), _i(0)
    st = lib().fa_tile_config(pass_, d, int(causal), ctypes.byref(bm), ctypes.byref(bn))
    return st, bm.value, bn.value


def fa_fwd_debug_visits(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, visited, stream):
    return lib().fa_fwd_debug_visits(q, k, v, o, lse, B, H, N, d, int(causal), scale, block_mask, visited,
                                     stream)


def fa_bwd_debug_visits(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, workspace,
                        workspace_bytes, visited_kv, visited_q, stream):
    return lib().fa_bwd_debug_visits(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, int(causal), scale,
                                     block_mask, workspace, workspace_bytes, visited_kv, visited_q, stream)


def fa_atomic_add_probe(dst, dst_floats, workgroups, reps, stream):
    return lib().fa_atomic_add_probe(dst, dst_floats, workgroups, reps, stream)


def fa_build_id() -> str:
    return lib().fa_build_id().decode()


def fa_status_str(status: int) -> str:
    try:
        return lib().fa_status_str(status).decode()
    except ImportError:
        return STATUS.get(status, "unknown")
