"""Python binding of libengram.so (ctypes; same names as the C ABI).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream.  Importing this
module loads the library and raises ImportError when it has not been built
(``python -m gram_hashed_embedding_amd.build``); there is no fallback path.

All calls are asynchronous on ``torch.cuda.current_stream()`` of the
tensors' device (or the stream passed in), exactly like the C entry points.
"""
from __future__ import annotations

import contextlib
import ctypes
import re
from pathlib import Path

import torch

from . import abi
from .abi import (ENGRAM_EALIGN, ENGRAM_EHIP, ENGRAM_EINVAL, ENGRAM_EWORKSPACE,  # noqa: F401
                  ENGRAM_OK, ERR_NO_PLAN, ERR_STALLED, MAX_HEADS, MAX_NGRAM,
                  NOALLOC_SCRATCH_BYTES, SCATTER_ATOMIC, SCATTER_ROWSPARSE, SCATTER_SORTED)

_PKG = Path(__file__).resolve().parent
LIBRARY = _PKG / "libengram.so"
HEADER = _PKG.parent / "include" / "engram.h"

if not LIBRARY.exists():
    raise ImportError(f"{LIBRARY} is missing: build it with "
                      "`python -m gram_hashed_embedding_amd.build` (hipcc, gfx950)")

_lib = abi.declare(ctypes.CDLL(str(LIBRARY)))


class EngramError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {engram_status_string(status)} (status {status})")


def engram_status_string(status: int) -> str:
    return _lib.engram_status_string(int(status)).decode()


def engram_abi_version() -> int:
    return int(_lib.engram_abi_version())


def declared_symbols() -> list[str]:
    """Names of the functions include/engram.h declares."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(engram_\w+)\s*\(", text,
                                 re.MULTILINE)))


def _check(status: int, call: str) -> None:
    if status != ENGRAM_OK:
        raise EngramError(status, call)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# Host arrays of hash constants, kept per value: the library only reads them
# during a call, so one array serves every call with the same constants and a
# step does not rebuild them (the per-call host cost bounds small steps).
_HOST_I64 = {}


def _host_i64(values, length, what):
    vals = tuple(values.tolist() if hasattr(values, "tolist") else values)
    if len(vals) != length:
        raise ValueError(f"{what} must have {length} entries, got {len(vals)}")
    arr = _HOST_I64.get(vals)
    if arr is None:
        arr = (ctypes.c_int64 * max(length, 1))(*(int(v) for v in vals))
        if len(_HOST_I64) >= 256:
            _HOST_I64.clear()
        _HOST_I64[vals] = arr
    return arr


_SAME_DEVICE = contextlib.nullcontext()


def _on(device):
    """Make `device` current for a call (no switch when it already is)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return _SAME_DEVICE
    return torch.cuda.device(device)


def _device_tensor(t, dtype, what):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a device (cuda) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    return t


def _stream(device, stream):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def engram_hash(tokens, ngram_size, heads_per_ngram, eos_id, multipliers, primes, offsets,
                table_rows, seq_ids=None, out=None, stream=None):
    """Row ids int64 [batch, seq, H] of tokens int64 [batch, seq]."""
    _device_tensor(tokens, torch.int64, "tokens")
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    batch, seq = tokens.shape
    if not 2 <= int(ngram_size) <= MAX_NGRAM:
        raise ValueError(f"ngram_size must be in [2, {MAX_NGRAM}]")
    heads = (int(ngram_size) - 1) * int(heads_per_ngram)
    if seq_ids is not None:
        _device_tensor(seq_ids, torch.int64, "seq_ids")
        if seq_ids.shape != tokens.shape:
            raise ValueError("seq_ids must have the shape of tokens")
    if out is None:
        out = torch.empty((batch, seq, heads), dtype=torch.int64, device=tokens.device)
    _device_tensor(out, torch.int64, "out")
    if out.numel() != batch * seq * heads:
        raise ValueError("out must hold batch * seq * H ids")
    mult = _host_i64(multipliers, int(ngram_size), "multipliers")
    pr = _host_i64(primes, heads, "primes")
    off = _host_i64(offsets, heads, "offsets")
    with _on(tokens.device):
        status = _lib.engram_hash(_ptr(tokens), _ptr(seq_ids), batch, seq, int(ngram_size),
                                  int(heads_per_ngram), int(eos_id), mult, pr, off,
                                  int(table_rows), _ptr(out), _stream(tokens.device, stream))
    _check(status, "engram_hash")
    return out


def engram_hash_slice(tokens, seq_start, seq_end, ngram_size, heads_per_ngram, eos_id,
                      multipliers, primes, offsets, table_rows, seq_ids=None, out=None,
                      stream=None):
    """Row ids int64 [batch, seq_end - seq_start, H] of positions
    [seq_start, seq_end) of the complete sequence tokens int64
    [batch, global_seq] (history may reach back before seq_start)."""
    _device_tensor(tokens, torch.int64, "tokens")
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, global_seq]")
    batch, gseq = tokens.shape
    start, end = int(seq_start), int(seq_end)
    if not 0 <= start <= end <= gseq:
        raise ValueError(f"slice [{start}, {end}) is not inside [0, {gseq})")
    if not 2 <= int(ngram_size) <= MAX_NGRAM:
        raise ValueError(f"ngram_size must be in [2, {MAX_NGRAM}]")
    heads = (int(ngram_size) - 1) * int(heads_per_ngram)
    if seq_ids is not None:
        _device_tensor(seq_ids, torch.int64, "seq_ids")
        if seq_ids.shape != tokens.shape:
            raise ValueError("seq_ids must have the shape of tokens")
    if out is None:
        out = torch.empty((batch, end - start, heads), dtype=torch.int64, device=tokens.device)
    _device_tensor(out, torch.int64, "out")
    if out.numel() != batch * (end - start) * heads:
        raise ValueError("out must hold batch * (seq_end - seq_start) * H ids")
    mult = _host_i64(multipliers, int(ngram_size), "multipliers")
    pr = _host_i64(primes, heads, "primes")
    off = _host_i64(offsets, heads, "offsets")
    with _on(tokens.device):
        status = _lib.engram_hash_slice(_ptr(tokens), _ptr(seq_ids), batch, gseq, start, end,
                                        int(ngram_size), int(heads_per_ngram), int(eos_id),
                                        mult, pr, off, int(table_rows), _ptr(out),
                                        _stream(tokens.device, stream))
    _check(status, "engram_hash_slice")
    return out


def forward_global_slice(tokens, seq_start, seq_end, table, ngram_size, heads_per_ngram,
                         eos_id, multipliers, primes, offsets, seq_ids=None, stream=None):
    """The slice's values bf16 [batch, seq_end - seq_start, H * head_dim]
    (engram_lookup_slice: one library call)."""
    out = engram_lookup_slice(tokens, seq_start, seq_end, table, ngram_size, heads_per_ngram,
                              eos_id, multipliers, primes, offsets, seq_ids=seq_ids,
                              stream=stream)
    return out.reshape(out.shape[0], out.shape[1], -1)


def engram_gather(row_ids, table, out=None, err_count=None, stream=None):
    """bf16 rows table[row_ids] with shape row_ids.shape + (head_dim,)."""
    _device_tensor(row_ids, torch.int64, "row_ids")
    _device_tensor(table, torch.bfloat16, "table")
    if table.dim() != 2:
        raise ValueError("table must be [rows, head_dim]")
    rows, dim = table.shape
    n = row_ids.numel()
    if out is None:
        out = torch.empty((*row_ids.shape, dim), dtype=torch.bfloat16, device=row_ids.device)
    _device_tensor(out, torch.bfloat16, "out")
    if out.numel() != n * dim:
        raise ValueError("out must hold n * head_dim values")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    with _on(row_ids.device):
        status = _lib.engram_gather(_ptr(row_ids), n, _ptr(table), rows, dim, _ptr(out),
                                    _ptr(err_count), _stream(row_ids.device, stream))
    _check(status, "engram_gather")
    return out


def engram_scatter_add_workspace(n, table_rows, head_dim, mode=SCATTER_SORTED) -> int:
    size = _lib.engram_scatter_add_workspace(int(n), int(table_rows), int(head_dim), int(mode))
    if size == ctypes.c_size_t(-1).value:
        raise EngramError(ENGRAM_EINVAL, "engram_scatter_add_workspace")
    return int(size)


def _workspace(workspace, n, table_rows, dim, mode, device):
    """The caller's workspace (the library checks its size), or a new one."""
    if workspace is None:
        need = engram_scatter_add_workspace(n, table_rows, dim, mode)
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=device)
    _device_tensor(workspace, torch.uint8, "workspace")
    return workspace


def engram_scatter_add(row_ids, grads, grad_table, mode=SCATTER_SORTED, workspace=None,
                       err_count=None, stream=None):
    """grad_table[r] += sum of grads[i] over row_ids[i] == r (in place)."""
    _device_tensor(row_ids, torch.int64, "row_ids")
    _device_tensor(grads, torch.bfloat16, "grads")
    _device_tensor(grad_table, torch.float32, "grad_table")
    rows, dim = grad_table.shape
    n = row_ids.numel()
    if grads.numel() != n * dim:
        raise ValueError("grads must hold n * head_dim values")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    ws = None
    if mode == SCATTER_SORTED:
        ws = _workspace(workspace, n, rows, dim, mode, row_ids.device)
    with _on(row_ids.device):
        status = _lib.engram_scatter_add(_ptr(row_ids), n, _ptr(grads), dim, _ptr(grad_table),
                                         rows, int(mode), _ptr(ws),
                                         0 if ws is None else ws.numel(), _ptr(err_count),
                                         _stream(row_ids.device, stream))
    _check(status, "engram_scatter_add")
    return grad_table


def engram_scatter_add_rowsparse(row_ids, grads, table_rows, unique_ids=None, unique_grads=None,
                                 num_unique=None, workspace=None, err_count=None, stream=None):
    """(unique_ids int64 [n], unique_grads fp32 [n, dim], num_unique int64 [1]);
    the first num_unique entries are valid (num_unique stays on the device)."""
    _device_tensor(row_ids, torch.int64, "row_ids")
    _device_tensor(grads, torch.bfloat16, "grads")
    n = row_ids.numel()
    dim = grads.shape[-1]
    if grads.numel() != n * dim:
        raise ValueError("grads must hold n * head_dim values")
    dev = row_ids.device
    if unique_ids is None:
        unique_ids = torch.empty(max(n, 1), dtype=torch.int64, device=dev)
    if unique_grads is None:
        unique_grads = torch.empty((max(n, 1), dim), dtype=torch.float32, device=dev)
    if num_unique is None:
        num_unique = torch.empty(1, dtype=torch.int64, device=dev)
    _device_tensor(unique_ids, torch.int64, "unique_ids")
    _device_tensor(unique_grads, torch.float32, "unique_grads")
    _device_tensor(num_unique, torch.int64, "num_unique")
    if unique_ids.numel() < n or unique_grads.numel() < n * dim:
        raise ValueError("unique_ids / unique_grads must hold n entries")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    ws = _workspace(workspace, n, table_rows, dim, SCATTER_ROWSPARSE, dev)
    with _on(dev):
        status = _lib.engram_scatter_add_rowsparse(_ptr(row_ids), n, _ptr(grads), dim,
                                                   int(table_rows), _ptr(unique_ids),
                                                   _ptr(unique_grads), _ptr(num_unique),
                                                   _ptr(ws), ws.numel(), _ptr(err_count),
                                                   _stream(dev, stream))
    _check(status, "engram_scatter_add_rowsparse")
    return unique_ids, unique_grads, num_unique


def engram_scatter_add_rowsparse_noalloc(row_ids, grads, table_rows, unique_ids, unique_grads,
                                         num_unique, err_count=None, stream=None):
    """engram_scatter_add_rowsparse with the library's fixed device array as
    its workspace: every output buffer is the caller's and nothing is
    allocated.  Raises EngramError (workspace) when n ids need more than
    NOALLOC_SCRATCH_BYTES of workspace.  Calls that overlap on one device race."""
    _device_tensor(row_ids, torch.int64, "row_ids")
    _device_tensor(grads, torch.bfloat16, "grads")
    n = row_ids.numel()
    dim = grads.shape[-1]
    if grads.numel() != n * dim:
        raise ValueError("grads must hold n * head_dim values")
    _device_tensor(unique_ids, torch.int64, "unique_ids")
    _device_tensor(unique_grads, torch.float32, "unique_grads")
    _device_tensor(num_unique, torch.int64, "num_unique")
    if unique_ids.numel() < n or unique_grads.numel() < n * dim:
        raise ValueError("unique_ids / unique_grads must hold n entries")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    dev = row_ids.device
    with _on(dev):
        status = _lib.engram_scatter_add_rowsparse_noalloc(
            _ptr(row_ids), n, _ptr(grads), dim, int(table_rows), _ptr(unique_ids),
            _ptr(unique_grads), _ptr(num_unique), _ptr(err_count), _stream(dev, stream))
    _check(status, "engram_scatter_add_rowsparse_noalloc")
    return unique_ids, unique_grads, num_unique


def engram_scatter_plan(row_ids, table_rows, head_dim, workspace=None, err_count=None,
                        stream=None):
    """Sort the row ids and slot their distinct rows into `workspace`
    (allocated when not given); returns the workspace."""
    _device_tensor(row_ids, torch.int64, "row_ids")
    n = row_ids.numel()
    ws = _workspace(workspace, n, table_rows, head_dim, SCATTER_ROWSPARSE, row_ids.device)
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    with _on(row_ids.device):
        status = _lib.engram_scatter_plan(_ptr(row_ids), n, int(table_rows), int(head_dim),
                                          _ptr(ws), ws.numel(), _ptr(err_count),
                                          _stream(row_ids.device, stream))
    _check(status, "engram_scatter_plan")
    return ws


def engram_scatter_apply(grads, workspace, table_rows, grad_table=None, unique_ids=None,
                         unique_grads=None, num_unique=None, err_count=None, stream=None):
    """Sums of `grads` (bf16 [n, head_dim]) per the plan in `workspace`: into
    grad_table (dense, in place) when given, else row-sparse (allocated when
    not given); returns grad_table or (unique_ids, unique_grads, num_unique).
    err_count (int64 [1] on the device) receives ERR_NO_PLAN when the
    workspace holds no complete plan of these sizes, ERR_STALLED for a plan
    whose wait expired (nothing is written then)."""
    _device_tensor(grads, torch.bfloat16, "grads")
    _device_tensor(workspace, torch.uint8, "workspace")
    dim = grads.shape[-1]
    n = grads.numel() // dim if dim else 0
    dev = grads.device
    if grad_table is not None:
        _device_tensor(grad_table, torch.float32, "grad_table")
        if grad_table.shape[-1] != dim:
            raise ValueError("grad_table width differs from the gradients")
    else:
        if unique_ids is None:
            unique_ids = torch.empty(max(n, 1), dtype=torch.int64, device=dev)
        if unique_grads is None:
            unique_grads = torch.empty((max(n, 1), dim), dtype=torch.float32, device=dev)
        if num_unique is None:
            num_unique = torch.empty(1, dtype=torch.int64, device=dev)
        _device_tensor(unique_ids, torch.int64, "unique_ids")
        _device_tensor(unique_grads, torch.float32, "unique_grads")
        _device_tensor(num_unique, torch.int64, "num_unique")
        if unique_ids.numel() < n or unique_grads.numel() < n * dim:
            raise ValueError("unique_ids / unique_grads must hold n entries")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    with _on(dev):
        status = _lib.engram_scatter_apply(_ptr(grads), n, dim, int(table_rows),
                                           _ptr(grad_table), _ptr(unique_ids),
                                           _ptr(unique_grads), _ptr(num_unique), _ptr(workspace),
                                           workspace.numel(), _ptr(err_count),
                                           _stream(dev, stream))
    _check(status, "engram_scatter_apply")
    if grad_table is not None:
        return grad_table
    return unique_ids, unique_grads, num_unique


def engram_signsgd_rowsparse(unique_ids, unique_grads, num_unique, table, lr, err_count=None,
                             stream=None):
    """SignSGD on the rows a row-sparse gradient lists, in place on the bf16
    table [rows, head_dim]; num_unique is the device count U."""
    _device_tensor(unique_ids, torch.int64, "unique_ids")
    _device_tensor(unique_grads, torch.float32, "unique_grads")
    _device_tensor(num_unique, torch.int64, "num_unique")
    _device_tensor(table, torch.bfloat16, "table")
    if table.dim() != 2:
        raise ValueError("table must be [rows, head_dim]")
    rows, dim = table.shape
    cap = unique_ids.numel()
    if unique_grads.numel() != cap * dim:
        raise ValueError("unique_grads must be [capacity, head_dim]")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    with _on(table.device):
        status = _lib.engram_signsgd_rowsparse(_ptr(unique_ids), _ptr(unique_grads),
                                               _ptr(num_unique), cap, dim, _ptr(table), rows,
                                               float(lr), _ptr(err_count),
                                               _stream(table.device, stream))
    _check(status, "engram_signsgd_rowsparse")
    return table


def engram_scatter_apply_signsgd(grads, workspace, table, lr, err_count=None, stream=None):
    """The planned backward of bf16 grads [n, head_dim] fused with one
    SignSGD step on the bf16 table (in place)."""
    _device_tensor(grads, torch.bfloat16, "grads")
    _device_tensor(workspace, torch.uint8, "workspace")
    _device_tensor(table, torch.bfloat16, "table")
    rows, dim = table.shape
    n = grads.numel() // dim
    if grads.numel() != n * dim:
        raise ValueError("grads must be [n, head_dim] with the table's head_dim")
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    with _on(table.device):
        status = _lib.engram_scatter_apply_signsgd(_ptr(grads), n, dim, rows, _ptr(table),
                                                   float(lr), _ptr(workspace),
                                                   workspace.numel(), _ptr(err_count),
                                                   _stream(table.device, stream))
    _check(status, "engram_scatter_apply_signsgd")
    return table


def engram_ple_conv(x, weight, dilation, bias=None, seq_ids=None, halo=None, out=None,
                    stream=None):
    """Causal dilated depthwise conv of bf16 x [batch, seq, channels] with
    weight [channels, K] (bf16), optional bias [channels], packed-segment ids
    [batch, halo + seq] and a halo [batch, halo, channels] of preceding
    positions; returns bf16 [batch, seq, channels]."""
    _device_tensor(x, torch.bfloat16, "x")
    _device_tensor(weight, torch.bfloat16, "weight")
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x.shape[2]:
        raise ValueError("x must be [batch, seq, channels] and weight [channels, K]")
    batch, seq, ch = x.shape
    hl = 0
    if halo is not None:
        _device_tensor(halo, torch.bfloat16, "halo")
        if halo.dim() != 3 or halo.shape[0] != batch or halo.shape[2] != ch:
            raise ValueError("halo must be [batch, halo_len, channels]")
        hl = halo.shape[1]
    if bias is not None:
        _device_tensor(bias, torch.bfloat16, "bias")
        if bias.numel() != ch:
            raise ValueError("bias must have one value per channel")
    if seq_ids is not None:
        _device_tensor(seq_ids, torch.int64, "seq_ids")
        if tuple(seq_ids.shape) != (batch, hl + seq):
            raise ValueError("seq_ids must be [batch, halo_len + seq]")
    if out is None:
        out = torch.empty_like(x)
    _device_tensor(out, torch.bfloat16, "out")
    if out.shape != x.shape:
        raise ValueError("out must have the shape of x")
    with _on(x.device):
        status = _lib.engram_ple_conv(_ptr(x), _ptr(halo), hl, _ptr(seq_ids), _ptr(weight),
                                      _ptr(bias), batch, seq, ch, weight.shape[1],
                                      int(dilation), _ptr(out), _stream(x.device, stream))
    _check(status, "engram_ple_conv")
    return out


def _hash_args(tokens, ngram_size, heads_per_ngram, multipliers, primes, offsets, seq_ids):
    _device_tensor(tokens, torch.int64, "tokens")
    if tokens.dim() != 2:
        raise ValueError("tokens must be [batch, seq]")
    if not 2 <= int(ngram_size) <= MAX_NGRAM:
        raise ValueError(f"ngram_size must be in [2, {MAX_NGRAM}]")
    heads = (int(ngram_size) - 1) * int(heads_per_ngram)
    if seq_ids is not None:
        _device_tensor(seq_ids, torch.int64, "seq_ids")
        if seq_ids.shape != tokens.shape:
            raise ValueError("seq_ids must have the shape of tokens")
    return (heads, _host_i64(multipliers, int(ngram_size), "multipliers"),
            _host_i64(primes, heads, "primes"), _host_i64(offsets, heads, "offsets"))


def engram_lookup(tokens, table, ngram_size, heads_per_ngram, eos_id, multipliers, primes,
                  offsets, seq_ids=None, out=None, row_ids=None, stream=None):
    """The forward in one pass: bf16 [batch, seq, H, head_dim] rows of the
    hashed ids of tokens int64 [batch, seq]; also writes the ids into row_ids
    (int64 [batch, seq, H]) when given."""
    heads, mult, pr, off = _hash_args(tokens, ngram_size, heads_per_ngram, multipliers, primes,
                                      offsets, seq_ids)
    _device_tensor(table, torch.bfloat16, "table")
    if table.dim() != 2:
        raise ValueError("table must be [rows, head_dim]")
    batch, seq = tokens.shape
    rows, dim = table.shape
    if out is None:
        out = torch.empty((batch, seq, heads, dim), dtype=torch.bfloat16, device=tokens.device)
    _device_tensor(out, torch.bfloat16, "out")
    if out.numel() != batch * seq * heads * dim:
        raise ValueError("out must hold batch * seq * H * head_dim values")
    if row_ids is not None:
        _device_tensor(row_ids, torch.int64, "row_ids")
        if row_ids.numel() != batch * seq * heads:
            raise ValueError("row_ids must hold batch * seq * H ids")
    with _on(tokens.device):
        status = _lib.engram_lookup(_ptr(tokens), _ptr(seq_ids), batch, seq, int(ngram_size),
                                    int(heads_per_ngram), int(eos_id), mult, pr, off,
                                    _ptr(table), rows, dim, _ptr(out), _ptr(row_ids),
                                    _stream(tokens.device, stream))
    _check(status, "engram_lookup")
    return out


def engram_lookup_slice(tokens, seq_start, seq_end, table, ngram_size, heads_per_ngram, eos_id,
                        multipliers, primes, offsets, seq_ids=None, out=None, row_ids=None,
                        stream=None):
    """engram_lookup for positions [seq_start, seq_end) of the complete
    sequence tokens int64 [batch, global_seq] (history may reach back before
    seq_start): bf16 [batch, seq_end - seq_start, H, head_dim]; also writes
    the ids into row_ids (int64 [batch, seq_end - seq_start, H]) when given."""
    heads, mult, pr, off = _hash_args(tokens, ngram_size, heads_per_ngram, multipliers, primes,
                                      offsets, seq_ids)
    _device_tensor(table, torch.bfloat16, "table")
    if table.dim() != 2:
        raise ValueError("table must be [rows, head_dim]")
    batch, gseq = tokens.shape
    start, end = int(seq_start), int(seq_end)
    if not 0 <= start <= end <= gseq:
        raise ValueError(f"slice [{start}, {end}) is not inside [0, {gseq})")
    local = end - start
    rows, dim = table.shape
    if out is None:
        out = torch.empty((batch, local, heads, dim), dtype=torch.bfloat16, device=tokens.device)
    _device_tensor(out, torch.bfloat16, "out")
    if out.numel() != batch * local * heads * dim:
        raise ValueError("out must hold batch * (seq_end - seq_start) * H * head_dim values")
    if row_ids is not None:
        _device_tensor(row_ids, torch.int64, "row_ids")
        if row_ids.numel() != batch * local * heads:
            raise ValueError("row_ids must hold batch * (seq_end - seq_start) * H ids")
    with _on(tokens.device):
        status = _lib.engram_lookup_slice(_ptr(tokens), _ptr(seq_ids), batch, gseq, start, end,
                                          int(ngram_size), int(heads_per_ngram), int(eos_id),
                                          mult, pr, off, _ptr(table), rows, dim, _ptr(out),
                                          _ptr(row_ids), _stream(tokens.device, stream))
    _check(status, "engram_lookup_slice")
    return out


def engram_scatter_plan_tokens(tokens, table_rows, head_dim, ngram_size, heads_per_ngram, eos_id,
                               multipliers, primes, offsets, seq_ids=None, workspace=None,
                               err_count=None, stream=None):
    """The backward's plan for the hashed ids of tokens, made from the tokens;
    returns the workspace (allocated when not given).  err_count (int64 [1]
    on the device) receives ERR_STALLED should a bounded wait expire."""
    heads, mult, pr, off = _hash_args(tokens, ngram_size, heads_per_ngram, multipliers, primes,
                                      offsets, seq_ids)
    batch, seq = tokens.shape
    n = batch * seq * heads
    ws = _workspace(workspace, n, table_rows, head_dim, SCATTER_ROWSPARSE, tokens.device)
    if err_count is not None:
        _device_tensor(err_count, torch.int64, "err_count")
    with _on(tokens.device):
        status = _lib.engram_scatter_plan_tokens(_ptr(tokens), _ptr(seq_ids), batch, seq,
                                                 int(ngram_size), int(heads_per_ngram),
                                                 int(eos_id), mult, pr, off, int(table_rows),
                                                 int(head_dim), _ptr(ws), ws.numel(),
                                                 _ptr(err_count), _stream(tokens.device, stream))
    _check(status, "engram_scatter_plan_tokens")
    return ws



# ---------------------------------------------------------------- schedules --
class Schedule:
    """A list of the library's calls and stream-event operations, built once
    and enqueued with one native call per run (engram_run_ops): what a
    training loop submits for a step, without the binding's and torch's
    per-call host cost each time.  Each method appends one operation with the
    arguments of the call of the same name (checked as that call checks
    them); ``stream`` defaults to the current stream when the operation is
    added.  The schedule holds raw pointers, so it keeps a reference to
    every tensor, constant array, stream and event it was given; a schedule
    must be rebuilt whenever one of them would be replaced."""

    def __init__(self):
        self._ops = []
        self._keep = []
        self._array = None

    def _add(self, keep, **fields):
        o = abi.EngramOp()
        for k, v in fields.items():
            setattr(o, k, v)
        self._ops.append(o)
        self._keep.extend(keep)
        self._array = None
        return self

    @staticmethod
    def _sp(device, stream):
        s = stream if stream is not None else torch.cuda.current_stream(device)
        return s, s.cuda_stream

    def lookup(self, tokens, table, ngram_size, heads_per_ngram, eos_id, multipliers, primes,
               offsets, out, seq_ids=None, row_ids=None, stream=None):
        heads, mult, pr, off = _hash_args(tokens, ngram_size, heads_per_ngram, multipliers,
                                          primes, offsets, seq_ids)
        _device_tensor(table, torch.bfloat16, "table")
        _device_tensor(out, torch.bfloat16, "out")
        if row_ids is not None:
            _device_tensor(row_ids, torch.int64, "row_ids")
        s, sp = self._sp(tokens.device, stream)
        batch, seq = tokens.shape
        return self._add(
            [tokens, seq_ids, table, out, row_ids, mult, pr, off, s],
            op=abi.OP_LOOKUP, stream=sp, d_tokens=tokens.data_ptr(),
            d_seq_ids=None if seq_ids is None else seq_ids.data_ptr(), batch=batch, seq=seq,
            ngram_size=int(ngram_size), heads_per_ngram=int(heads_per_ngram),
            eos_id=int(eos_id), h_multipliers=mult, h_primes=pr, h_offsets=off,
            d_table=table.data_ptr(), table_rows=table.shape[0], head_dim=table.shape[1],
            d_out=out.data_ptr(), d_row_ids=None if row_ids is None else row_ids.data_ptr())

    def plan_tokens(self, tokens, table_rows, head_dim, ngram_size, heads_per_ngram, eos_id,
                    multipliers, primes, offsets, workspace, seq_ids=None, err_count=None,
                    stream=None):
        heads, mult, pr, off = _hash_args(tokens, ngram_size, heads_per_ngram, multipliers,
                                          primes, offsets, seq_ids)
        _device_tensor(workspace, torch.uint8, "workspace")
        if err_count is not None:
            _device_tensor(err_count, torch.int64, "err_count")
        s, sp = self._sp(tokens.device, stream)
        batch, seq = tokens.shape
        return self._add(
            [tokens, seq_ids, workspace, err_count, mult, pr, off, s],
            op=abi.OP_PLAN_TOKENS, stream=sp, d_tokens=tokens.data_ptr(),
            d_seq_ids=None if seq_ids is None else seq_ids.data_ptr(), batch=batch, seq=seq,
            ngram_size=int(ngram_size), heads_per_ngram=int(heads_per_ngram),
            eos_id=int(eos_id), h_multipliers=mult, h_primes=pr, h_offsets=off,
            table_rows=int(table_rows), head_dim=int(head_dim),
            d_workspace=workspace.data_ptr(), workspace_bytes=workspace.numel(),
            d_err_count=None if err_count is None else err_count.data_ptr())

    def apply(self, grads, workspace, table_rows, grad_table=None, unique_ids=None,
              unique_grads=None, num_unique=None, err_count=None, stream=None):
        _device_tensor(grads, torch.bfloat16, "grads")
        _device_tensor(workspace, torch.uint8, "workspace")
        for t, dt, what in ((grad_table, torch.float32, "grad_table"),
                            (unique_ids, torch.int64, "unique_ids"),
                            (unique_grads, torch.float32, "unique_grads"),
                            (num_unique, torch.int64, "num_unique"),
                            (err_count, torch.int64, "err_count")):
            if t is not None:
                _device_tensor(t, dt, what)
        s, sp = self._sp(grads.device, stream)
        p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
        return self._add(
            [grads, workspace, grad_table, unique_ids, unique_grads, num_unique, err_count, s],
            op=abi.OP_APPLY, stream=sp, d_grads=grads.data_ptr(), n=grads.shape[0],
            head_dim=grads.shape[1], table_rows=int(table_rows),
            d_grad_table=p(grad_table), d_unique_ids=p(unique_ids),
            d_unique_grads=p(unique_grads), d_num_unique=p(num_unique),
            d_workspace=workspace.data_ptr(), workspace_bytes=workspace.numel(),
            d_err_count=p(err_count))

    def apply_signsgd(self, grads, workspace, table, lr, err_count=None, stream=None):
        _device_tensor(grads, torch.bfloat16, "grads")
        _device_tensor(workspace, torch.uint8, "workspace")
        _device_tensor(table, torch.bfloat16, "table")
        if err_count is not None:
            _device_tensor(err_count, torch.int64, "err_count")
        s, sp = self._sp(grads.device, stream)
        return self._add(
            [grads, workspace, table, err_count, s],
            op=abi.OP_APPLY_SIGNSGD, stream=sp, d_grads=grads.data_ptr(), n=grads.shape[0],
            head_dim=grads.shape[1], table_rows=table.shape[0], d_table_rw=table.data_ptr(),
            lr=float(lr), d_workspace=workspace.data_ptr(), workspace_bytes=workspace.numel(),
            d_err_count=None if err_count is None else err_count.data_ptr())

    def _event_op(self, op, event, stream):
        s, sp = self._sp(torch.device("cuda", torch.cuda.current_device()), stream)
        if not event.cuda_event:  # torch creates an event when it is first recorded
            event.record(s)
        return self._add([event, s], op=op, stream=sp, event=event.cuda_event)

    def record(self, event, stream=None):
        """event.record(stream), in the schedule."""
        return self._event_op(abi.OP_RECORD, event, stream)

    def wait(self, event, stream=None):
        """stream.wait_event(event), in the schedule."""
        return self._event_op(abi.OP_WAIT, event, stream)

    def __len__(self):
        return len(self._ops)

    def run(self):
        """Enqueue every operation, in order (engram_run_ops)."""
        if self._array is None:
            self._array = (abi.EngramOp * max(len(self._ops), 1))(*self._ops)
        failed = ctypes.c_int64(-1)
        status = _lib.engram_run_ops(self._array, len(self._ops), ctypes.byref(failed))
        if status != ENGRAM_OK:
            raise EngramError(status, f"engram_run_ops (operation {failed.value})")
