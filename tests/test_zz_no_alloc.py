"""The allocation-free row-sparse scatter-add, called through the C ABI,
against engram_scatter_add_rowsparse (the same sums with a caller's
workspace), bit for bit: two calls in a row, the second smaller, so what the
first call leaves in the library's fixed array must not leak into the second."""
import ctypes

import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import engram as E

pytestmark = pytest.mark.gpu


def _ids(n, rows, seed):
    rng = np.random.default_rng(seed)
    ids = (rng.zipf(1.2, n) % rows).astype(np.int64)   # hot rows repeat
    ids[rng.random(n) < 0.01] = -1                       # padding
    ids[rng.random(n) < 0.001] = rows + 7                # invalid: counted
    return ids


def _noalloc(ids, grads, rows, dev):
    n, dim = grads.shape
    uid = torch.full((n,), -5, dtype=torch.int64, device=dev)
    uval = torch.full((n, dim), -5.0, dtype=torch.float32, device=dev)
    cnt = torch.full((1,), -5, dtype=torch.int64, device=dev)
    err = torch.zeros(1, dtype=torch.int64, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    status = E._lib.engram_scatter_add_rowsparse_noalloc(
        ctypes.c_void_p(ids.data_ptr()), n, ctypes.c_void_p(grads.data_ptr()), dim, rows,
        ctypes.c_void_p(uid.data_ptr()), ctypes.c_void_p(uval.data_ptr()),
        ctypes.c_void_p(cnt.data_ptr()), ctypes.c_void_p(err.data_ptr()), stream)
    assert status == E.ENGRAM_OK, E.engram_status_string(status)
    return uid, uval, cnt, err


def _with_workspace(ids, grads, rows, dev):
    err = torch.zeros(1, dtype=torch.int64, device=dev)
    uid, uval, cnt = E.engram_scatter_add_rowsparse(ids, grads, rows, err_count=err)
    return uid, uval, cnt, err


def _same(a, b):
    ua, ub = int(a[2].item()), int(b[2].item())
    assert ua == ub
    assert torch.equal(a[0][:ua], b[0][:ub])
    assert torch.equal(a[1][:ua].view(torch.int32), b[1][:ub].view(torch.int32))
    assert int(a[3].item()) == int(b[3].item())
    return ua


def test_noalloc_matches_workspace_call_twice():
    dev = torch.device("cuda:0")
    cases = [(300_000, 64, 2_000_000, 11), (7_001, 256, 50_000, 12)]   # second call smaller
    for n, dim, rows, seed in cases:
        print(f"noalloc case n={n} dim={dim} rows={rows}", flush=True)
        need = E.engram_scatter_add_workspace(n, rows, dim, E.SCATTER_ROWSPARSE)
        assert need <= E.NOALLOC_SCRATCH_BYTES
        ids = torch.from_numpy(_ids(n, rows, seed)).to(dev)
        g = torch.Generator(device=dev).manual_seed(seed)
        grads = torch.randn((n, dim), generator=g, device=dev).to(torch.bfloat16)
        got = _noalloc(ids, grads, rows, dev)
        want = _with_workspace(ids, grads, rows, dev)
        torch.cuda.synchronize()
        u = _same(got, want)
        assert 0 < u < n
        assert int(got[3].item()) > 0          # the invalid ids were counted
        # entries past U are untouched
        assert bool((got[0][u:] == -5).all())

