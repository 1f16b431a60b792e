"""ctypes front end of the C oracle (``engram_oracle.c``).

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It never
imports the product package and the product package never imports it.

All arrays are host numpy arrays.  bf16 data travels as ``uint16`` bit
patterns so that nothing here depends on a bf16 numpy dtype.  See the C
source for the citation of every step and the readings it takes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
SOURCE = _HERE / "engram_oracle.c"
LIBRARY = _HERE / "libengram_oracle.so"
# the same source built with -fopenmp: the all-core CPU baseline
LIBRARY_OMP = _HERE / "libengram_oracle_omp.so"
OMP_FLAGS = ("-fopenmp",)

_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)


def build(source: Path = SOURCE, output: Path = LIBRARY, extra_flags=()) -> Path:
    """Compile the oracle with gcc into a shared library and return its path."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
           *extra_flags, str(source), "-o", str(output)]
    subprocess.run(cmd, check=True)
    return output


def _ptr(arr, ctype):
    return arr.ctypes.data_as(ctype) if arr is not None else None


class Oracle:
    """One loaded copy of the oracle library."""

    @property
    def threads(self) -> int:
        """Threads its parallel loops use (1 for the serial build)."""
        return int(self._lib.oracle_threads())

    def __init__(self, library: Path | str = LIBRARY):
        self.path = str(library)
        lib = ctypes.CDLL(self.path)
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_hash.restype = ctypes.c_int
        lib.oracle_hash.argtypes = [_i64p, _i64p, ctypes.c_int64, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                    _i64p, _i64p, _i64p, _i64p]
        lib.oracle_gather.restype = ctypes.c_int64
        lib.oracle_gather.argtypes = [_i64p, ctypes.c_int64, _u16p, ctypes.c_int64,
                                      ctypes.c_int64, _u16p]
        lib.oracle_scatter_add_dense.restype = ctypes.c_int64
        lib.oracle_scatter_add_dense.argtypes = [_i64p, ctypes.c_int64, _u16p,
                                                 ctypes.c_int64, _f32p, ctypes.c_int64]
        lib.oracle_scatter_add_rowsparse.restype = ctypes.c_int64
        lib.oracle_scatter_add_rowsparse.argtypes = [_i64p, ctypes.c_int64, _u16p,
                                                     ctypes.c_int64, ctypes.c_int64,
                                                     _i64p, _f32p, _i64p]
        lib.oracle_ple_conv.restype = ctypes.c_int
        lib.oracle_ple_conv.argtypes = [_u16p, _u16p, ctypes.c_int64, _i64p, _u16p, _u16p,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_int, _u16p]
        lib.oracle_signsgd_rowsparse.restype = ctypes.c_int64
        lib.oracle_signsgd_rowsparse.argtypes = [_i64p, _f32p, ctypes.c_int64, ctypes.c_int64,
                                                 _u16p, ctypes.c_int64, ctypes.c_float]
        self._lib = lib

    # -- hash ---------------------------------------------------------------
    def hash(self, tokens, ngram_size, heads_per_ngram, eos_id, multipliers,
             primes, offsets, seq_ids=None):
        """Row IDs int64 [batch, seq, H] for tokens int64 [batch, seq]."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        if tokens.ndim != 2:
            raise ValueError("tokens must be [batch, seq]")
        batch, seq = tokens.shape
        heads = (ngram_size - 1) * heads_per_ngram
        mult = np.ascontiguousarray(multipliers, dtype=np.int64)
        pr = np.ascontiguousarray(primes, dtype=np.int64)
        off = np.ascontiguousarray(offsets, dtype=np.int64)
        if mult.shape != (ngram_size,) or pr.shape != (heads,) or off.shape != (heads,):
            raise ValueError("multipliers/primes/offsets have the wrong length")
        seg = None
        if seq_ids is not None:
            seg = np.ascontiguousarray(seq_ids, dtype=np.int64)
            if seg.shape != tokens.shape:
                raise ValueError("seq_ids must match tokens")
        out = np.empty((batch, seq, heads), dtype=np.int64)
        rc = self._lib.oracle_hash(_ptr(tokens, _i64p), _ptr(seg, _i64p), batch, seq,
                                   int(ngram_size), int(heads_per_ngram), int(eos_id),
                                   _ptr(mult, _i64p), _ptr(pr, _i64p), _ptr(off, _i64p),
                                   _ptr(out, _i64p))
        if rc != 0:
            raise ValueError("oracle_hash rejected its arguments")
        return out

    def hash_global_slice(self, tokens, seq_start, seq_end, ngram_size, heads_per_ngram,
                          eos_id, multipliers, primes, offsets, seq_ids=None):
        """Row IDs int64 [batch, seq_end - seq_start, H] of one slice of a
        complete sequence.  Follows the NeMo AutoModel v0.7 API page
        (qwen3_8_flash_next.engram), Qwen3_8_FlashNextNGramEmbedding.
        _forward_global_slice: the whole replicated sequence is hashed, then
        the positions [seq_start, seq_end) are kept."""
        tokens = np.asarray(tokens)
        if not 0 <= seq_start <= seq_end <= tokens.shape[1]:
            raise ValueError("slice outside the sequence")
        full = self.hash(tokens, ngram_size, heads_per_ngram, eos_id, multipliers, primes,
                         offsets, seq_ids=seq_ids)
        return full[:, seq_start:seq_end, :].copy()

    # -- gather -------------------------------------------------------------
    def gather(self, row_ids, table_bits):
        """(out uint16 [n, dim], invalid count) for table uint16 [rows, dim]."""
        ids = np.ascontiguousarray(row_ids, dtype=np.int64).reshape(-1)
        table = np.ascontiguousarray(table_bits, dtype=np.uint16)
        rows, dim = table.shape
        out = np.empty((ids.size, dim), dtype=np.uint16)
        bad = self._lib.oracle_gather(_ptr(ids, _i64p), ids.size, _ptr(table, _u16p),
                                      rows, dim, _ptr(out, _u16p))
        return out, int(bad)

    # -- scatter-add ----------------------------------------------------------
    def scatter_add_dense(self, row_ids, grad_bits, grad_table, inplace=False):
        """Accumulate into a copy of grad_table float32 [rows, dim] (into
        grad_table itself when inplace, which must then be a C-contiguous
        float32 array); returns (new table, invalid count)."""
        ids = np.ascontiguousarray(row_ids, dtype=np.int64).reshape(-1)
        grads = np.ascontiguousarray(grad_bits, dtype=np.uint16).reshape(ids.size, -1)
        if inplace:
            if grad_table.dtype != np.float32 or not grad_table.flags.c_contiguous:
                raise ValueError("an in-place table must be C-contiguous float32")
            table = grad_table
        else:
            table = np.array(grad_table, dtype=np.float32, copy=True, order="C")
        rows, dim = table.shape
        if grads.shape[1] != dim:
            raise ValueError("grad width differs from table width")
        bad = self._lib.oracle_scatter_add_dense(_ptr(ids, _i64p), ids.size,
                                                 _ptr(grads, _u16p), dim,
                                                 _ptr(table, _f32p), rows)
        if bad < 0:
            raise MemoryError("oracle_scatter_add_dense ran out of memory")
        return table, int(bad)

    def scatter_add_rowsparse(self, row_ids, grad_bits, dim, table_rows):
        """(unique ids int64 [U], sums float32 [U, dim], invalid count)."""
        ids = np.ascontiguousarray(row_ids, dtype=np.int64).reshape(-1)
        grads = np.ascontiguousarray(grad_bits, dtype=np.uint16).reshape(ids.size, dim)
        uid = np.empty(max(ids.size, 1), dtype=np.int64)
        vals = np.empty((max(ids.size, 1), dim), dtype=np.float32)
        count = np.zeros(1, dtype=np.int64)
        bad = self._lib.oracle_scatter_add_rowsparse(_ptr(ids, _i64p), ids.size,
                                                     _ptr(grads, _u16p), dim, table_rows,
                                                     _ptr(uid, _i64p), _ptr(vals, _f32p),
                                                     _ptr(count, _i64p))
        if bad < 0:
            raise MemoryError("oracle_scatter_add_rowsparse ran out of memory")
        u = int(count[0])
        return uid[:u].copy(), vals[:u].copy(), int(bad)

    # -- optimizer step -------------------------------------------------------
    def signsgd_rowsparse(self, unique_ids, unique_grads, table_bits, lr):
        """SignSGD on the listed rows of a copy of the bf16 table (uint16
        [rows, dim]); returns (new table bits, invalid count)."""
        ids = np.ascontiguousarray(unique_ids, dtype=np.int64).reshape(-1)
        table = np.array(table_bits, dtype=np.uint16, copy=True, order="C")
        rows, dim = table.shape
        grads = np.ascontiguousarray(unique_grads, dtype=np.float32).reshape(ids.size, dim)
        bad = self._lib.oracle_signsgd_rowsparse(_ptr(ids, _i64p), _ptr(grads, _f32p),
                                                 ids.size, dim, _ptr(table, _u16p), rows,
                                                 float(lr))
        return table, int(bad)


    # -- PLE convolution ------------------------------------------------------
    def ple_conv(self, x_bits, weight_bits, dilation, bias_bits=None, seq_ids=None,
                 halo_bits=None):
        """Causal depthwise conv with per-segment zero history: x uint16
        (bf16 bits) [batch, seq, channels], weight [channels, K], bias
        [channels] or None, seq_ids int64 [batch, halo + seq] or None, halo
        [batch, halo, channels] or None; returns uint16 [batch, seq, channels]."""
        x = np.ascontiguousarray(x_bits, dtype=np.uint16)
        batch, seq, channels = x.shape
        w = np.ascontiguousarray(weight_bits, dtype=np.uint16)
        if w.ndim != 2 or w.shape[0] != channels:
            raise ValueError("weight must be [channels, K]")
        K = w.shape[1]
        bias = None if bias_bits is None else np.ascontiguousarray(bias_bits, dtype=np.uint16)
        halo = None if halo_bits is None else np.ascontiguousarray(halo_bits, dtype=np.uint16)
        hl = 0 if halo is None else halo.shape[1]
        seg = None if seq_ids is None else np.ascontiguousarray(seq_ids, dtype=np.int64)
        if seg is not None and seg.shape != (batch, hl + seq):
            raise ValueError("seq_ids must be [batch, halo + seq]")
        out = np.empty_like(x)
        rc = self._lib.oracle_ple_conv(_ptr(x, _u16p), _ptr(halo, _u16p), hl, _ptr(seg, _i64p),
                                       _ptr(w, _u16p), _ptr(bias, _u16p), batch, seq, channels,
                                       K, int(dilation), _ptr(out, _u16p))
        if rc != 0:
            raise ValueError("oracle_ple_conv rejected its arguments")
        return out


_default = None
_default_omp = None


def default_oracle() -> Oracle:
    """The oracle built from this directory's source (built on first use if
    the library is missing or older than its source)."""
    global _default
    if _default is None:
        if (not LIBRARY.exists()
                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        _default = Oracle(LIBRARY)
    return _default


def build_all() -> None:
    """Both builds of the oracle: serial, and with OpenMP."""
    build()
    build(SOURCE, LIBRARY_OMP, OMP_FLAGS)


def openmp_oracle() -> Oracle:
    """The oracle built with OpenMP (its parallel loops on every thread
    OMP_NUM_THREADS allows); built on first use like default_oracle."""
    global _default_omp
    if _default_omp is None:
        if (not LIBRARY_OMP.exists()
                or os.path.getmtime(LIBRARY_OMP) < os.path.getmtime(SOURCE)):
            build(SOURCE, LIBRARY_OMP, OMP_FLAGS)
        _default_omp = Oracle(LIBRARY_OMP)
    return _default_omp
