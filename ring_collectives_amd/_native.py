"""ctypes loader for libring_collectives.so (argument marshalling only).

The library must have been built (``python -m ring_collectives_amd.build`` or
``__graft_entry__.build()``); if it is missing this module raises instead of
falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libring_collectives.so")

# ring_dtype_t / ring_op_t / error codes, as declared in include/ring_collectives.h
RING_F32, RING_BF16, RING_I32 = 0, 1, 2
(OP_PPERMUTE, OP_REDUCE_SCATTER, OP_ALL_GATHER, OP_ALL_REDUCE, OP_GEMM_REDUCE_SCATTER,
 OP_REDUCE_SCATTER_BIDIR, OP_ALL_GATHER_GEMM, OP_PSUM_CIRCULATING) = range(8)
RING_OK, RING_EINVAL, RING_EUNSUPPORTED, RING_EWORKSPACE, RING_EHIP, RING_ETIMEOUT, RING_EPROTOCOL = (
    0, -1, -2, -3, -4, -5, -6)
MAX_RANKS = 64
NOALLOC_SCRATCH_BYTES = 16 << 20   # RING_NOALLOC_SCRATCH_BYTES

_vp = ctypes.c_void_p
_pp = ctypes.POINTER(ctypes.c_void_p)
_sz = ctypes.c_size_t
_i = ctypes.c_int

SIGNATURES = {
    "ring_workspace_bytes": (_sz, [_i, _i, _sz, _i]),
    "ring_workspace_init": (_i, [_vp, _sz, _vp]),
    "ring_ppermute": (_i, [_pp, _pp, _i, _sz, _i, _vp]),
    "ring_reduce_scatter": (_i, [_pp, _pp, _i, _sz, _i, _vp, _sz, _vp]),
    "ring_reduce_scatter_bidir": (_i, [_pp, _pp, _i, _sz, _i, _vp, _sz, _vp]),
    "ring_psum_circulating": (_i, [_pp, _pp, _i, _sz, _i, _vp, _sz, _vp]),
    "ring_all_gather": (_i, [_pp, _pp, _i, _sz, _i, _vp, _sz, _vp]),
    "ring_all_reduce": (_i, [_pp, _pp, _i, _sz, _i, _vp, _sz, _vp]),
    "ring_all_reduce_noalloc": (_i, [_pp, _pp, _i, _sz, _i, _vp]),
    "gemm_reduce_scatter": (_i, [_pp, _pp, _pp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "all_gather_gemm": (_i, [_pp, _pp, _pp, _pp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "tp_mlp_layer": (_i, [_pp, _pp, _pp, _pp, _pp, _pp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "tp_mlp_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "ring_last_error": (_i, [_vp, _sz, _vp, ctypes.POINTER(ctypes.c_int)]),
    "ring_strerror": (ctypes.c_char_p, [_i]),
}

class Tuning(ctypes.Structure):
    """ring_tuning_t"""
    _fields_ = [("tile_vecs", ctypes.c_int), ("waves_per_cu", ctypes.c_int),
                ("map_mode", ctypes.c_int), ("timeout_s", ctypes.c_double),
                ("stepwise", ctypes.c_int), ("drop_round", ctypes.c_int),
                ("gemm_tile_n", ctypes.c_int), ("ll_max_chunk_bytes", ctypes.c_int),
                ("check_flags", ctypes.c_int)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


SIGNATURES["ring_get_tuning"] = (None, [ctypes.POINTER(Tuning)])
SIGNATURES["ring_set_tuning"] = (_i, [ctypes.POINTER(Tuning)])

_lib = None


class RingError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__("%s failed: %s (%d)" % (where, strerror(code), code))


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                "libring_collectives.so is not built (expected at %s); run "
                "`python -m ring_collectives_amd.build`" % LIB_PATH)
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def strerror(code: int) -> str:
    return lib().ring_strerror(code).decode()


def ptr_array(ptrs):
    """Host array of device pointers (void* const*).  ctypes passes the
    array itself for a pointer argument; it is returned twice so callers keep
    it alive while the call runs."""
    arr = (ctypes.c_void_p * max(len(ptrs), 1))(*ptrs)
    return arr, arr


def check(code: int, where: str) -> None:
    if code != RING_OK:
        raise RingError(code, where)


def get_tuning() -> dict:
    t = Tuning()
    lib().ring_get_tuning(ctypes.byref(t))
    return t.as_dict()


def set_tuning(**kw) -> dict:
    """Update tuning knobs; returns the previous values."""
    old = get_tuning()
    t = Tuning(**{**old, **kw})
    check(lib().ring_set_tuning(ctypes.byref(t)), "ring_set_tuning")
    return old
