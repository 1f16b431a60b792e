"""ctypes declarations of the libengram.so C ABI (include/engram.h), without
torch: the binding (engram.py) applies them to the built library, and the
host-side checks of the same entry points, built for the CPU under
sanitizers, are driven through them by the tests.
"""
from __future__ import annotations

import ctypes

ENGRAM_OK = 0
ENGRAM_EINVAL = -1
ENGRAM_EALIGN = -2
ENGRAM_EWORKSPACE = -3
ENGRAM_EHIP = -4
SCATTER_SORTED = 0
SCATTER_ATOMIC = 1
SCATTER_ROWSPARSE = 2
MAX_NGRAM = 8
MAX_HEADS = 64
NOALLOC_SCRATCH_BYTES = 64 << 20  # ENGRAM_NOALLOC_SCRATCH_BYTES
ERR_STALLED = 1 << 40             # ENGRAM_ERR_STALLED
ERR_NO_PLAN = 1 << 41             # ENGRAM_ERR_NO_PLAN

_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


def declare(lib):
    """Set the argument and result types of every entry point on `lib` (a
    ctypes.CDLL of libengram.so, or of a build of its host side); returns it."""
    lib.engram_status_string.restype = ctypes.c_char_p
    lib.engram_status_string.argtypes = [ctypes.c_int]
    lib.engram_abi_version.restype = ctypes.c_int
    lib.engram_abi_version.argtypes = []
    lib.engram_hash.restype = ctypes.c_int
    lib.engram_hash.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_int64, _i64p, _i64p, _i64p,
                                ctypes.c_int64, _vp, _vp]
    lib.engram_hash_slice.restype = ctypes.c_int
    lib.engram_hash_slice.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_int64, _i64p, _i64p, _i64p, ctypes.c_int64, _vp,
                                      _vp]
    lib.engram_lookup.restype = ctypes.c_int
    lib.engram_lookup.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int64, _i64p, _i64p, _i64p, _vp,
                                  ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]
    lib.engram_lookup_slice.restype = ctypes.c_int
    lib.engram_lookup_slice.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int64, _i64p, _i64p, _i64p, _vp, ctypes.c_int64,
                                        ctypes.c_int64, _vp, _vp, _vp]
    lib.engram_scatter_plan_tokens.restype = ctypes.c_int
    lib.engram_scatter_plan_tokens.argtypes = [_vp, _vp, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                               _i64p, _i64p, _i64p, ctypes.c_int64,
                                               ctypes.c_int64, _vp, ctypes.c_size_t, _vp, _vp]
    lib.engram_gather.restype = ctypes.c_int
    lib.engram_gather.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64, ctypes.c_int64, _vp,
                                  _vp, _vp]
    lib.engram_scatter_add_workspace.restype = ctypes.c_size_t
    lib.engram_scatter_add_workspace.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int32]
    lib.engram_scatter_add.restype = ctypes.c_int
    lib.engram_scatter_add.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64, _vp,
                                       ctypes.c_int64, ctypes.c_int32, _vp, ctypes.c_size_t, _vp,
                                       _vp]
    lib.engram_scatter_add_rowsparse.restype = ctypes.c_int
    lib.engram_scatter_add_rowsparse.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                                 ctypes.c_int64, _vp, _vp, _vp, _vp,
                                                 ctypes.c_size_t, _vp, _vp]

    lib.engram_scatter_add_rowsparse_noalloc.restype = ctypes.c_int
    lib.engram_scatter_add_rowsparse_noalloc.argtypes = [_vp, ctypes.c_int64, _vp, ctypes.c_int64,
                                                         ctypes.c_int64, _vp, _vp, _vp, _vp, _vp]

    lib.engram_scatter_plan.restype = ctypes.c_int
    lib.engram_scatter_plan.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp,
                                        ctypes.c_size_t, _vp, _vp]
    lib.engram_scatter_apply.restype = ctypes.c_int
    lib.engram_scatter_apply.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _vp,
                                         _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp]
    lib.engram_signsgd_rowsparse.restype = ctypes.c_int
    lib.engram_signsgd_rowsparse.argtypes = [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int64, _vp,
                                             ctypes.c_int64, ctypes.c_float, _vp, _vp]
    lib.engram_scatter_apply_signsgd.restype = ctypes.c_int
    lib.engram_scatter_apply_signsgd.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_int64, _vp, ctypes.c_float, _vp,
                                                 ctypes.c_size_t, _vp, _vp]
    lib.engram_ple_conv.restype = ctypes.c_int
    lib.engram_ple_conv.argtypes = [_vp, _vp, ctypes.c_int64, _vp, _vp, _vp, ctypes.c_int64,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    _vp, _vp]
    return lib
