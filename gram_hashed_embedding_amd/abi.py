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
ABI_VERSION = 3                   # ENGRAM_ABI_VERSION
OP_LOOKUP = 1                     # ENGRAM_OP_*
OP_PLAN_TOKENS = 2
OP_APPLY = 3
OP_APPLY_SIGNSGD = 4
OP_RECORD = 5
OP_WAIT = 6

_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p


class EngramOp(ctypes.Structure):
    """struct engram_op of include/engram.h, field for field."""
    _fields_ = [
        ("op", ctypes.c_int32), ("ngram_size", ctypes.c_int32),
        ("heads_per_ngram", ctypes.c_int32), ("lr", ctypes.c_float),
        ("stream", _vp), ("event", _vp),
        ("d_tokens", _vp), ("d_seq_ids", _vp),
        ("batch", ctypes.c_int64), ("seq", ctypes.c_int64), ("eos_id", ctypes.c_int64),
        ("h_multipliers", _i64p), ("h_primes", _i64p), ("h_offsets", _i64p),
        ("table_rows", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("d_table", _vp), ("d_out", _vp), ("d_row_ids", _vp),
        ("d_workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("d_grads", _vp), ("n", ctypes.c_int64),
        ("d_grad_table", _vp), ("d_unique_ids", _vp), ("d_unique_grads", _vp),
        ("d_num_unique", _vp),
        ("d_table_rw", _vp), ("d_err_count", _vp),
    ]


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

    lib.engram_run_ops.restype = ctypes.c_int
    lib.engram_run_ops.argtypes = [ctypes.POINTER(EngramOp), ctypes.c_int64, _i64p]

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
