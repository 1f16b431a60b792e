"""The apply reads a workspace only when it holds a complete plan of the
apply's n and table_rows, none of whose bounded waits expired; otherwise it
writes nothing (U = 0) and reports it in the error counter.  Every case keeps
its outputs inside larger allocations, so a write past a guard would show as
changed guard values, not as a fault; the inputs that would mislead an
unguarded apply stay inside their allocations too."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

DIM = 64


def _ids(n, rows, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return torch.from_numpy((rng.zipf(1.3, n) % rows).astype(np.int64)).to("cuda")


def _sparse_out(n):
    """Row-sparse outputs of capacity n inside twice that, filled with a guard value."""
    uid = torch.full((2 * n,), -7, dtype=torch.int64, device="cuda")
    val = torch.full((2 * n, DIM), -7.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((1,), -7, dtype=torch.int64, device="cuda")
    return uid, val, cnt


def _apply_sparse(grads, ws, rows, n):
    uid, val, cnt = _sparse_out(n)
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    E.engram_scatter_apply(grads, ws, rows, unique_ids=uid[:n], unique_grads=val[:n],
                           num_unique=cnt, err_count=err)
    torch.cuda.synchronize()
    return uid, val, int(cnt.item()), int(err.item())


def _untouched(uid, val):
    return bool((uid == -7).all()) and bool((val == -7.0).all())


def test_no_plan_in_workspace():
    n, rows = 20_000, 50_000
    grads = workloads.make_grads(n, DIM, 1, "cuda")
    size = E.engram_scatter_add_workspace(n, rows, DIM, E.SCATTER_ROWSPARSE)
    for fill in ("zeros", "random"):
        ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
        if fill == "random":
            ws = torch.randint(0, 256, (size,), dtype=torch.uint8, device="cuda",
                               generator=torch.Generator(device="cuda").manual_seed(3))
        uid, val, u, err = _apply_sparse(grads, ws, rows, n)
        assert u == 0 and err in (E.ERR_NO_PLAN, E.ERR_STALLED), (fill, err)
        assert _untouched(uid, val)
        # dense: the fp32 table is a view inside a larger guard-filled one
        big = torch.full((2 * rows, DIM), 3.0, dtype=torch.float32, device="cuda")
        derr = torch.zeros(1, dtype=torch.int64, device="cuda")
        E.engram_scatter_apply(grads, ws, rows, grad_table=big[:rows], err_count=derr)
        torch.cuda.synchronize()
        assert int(derr.item()) in (E.ERR_NO_PLAN, E.ERR_STALLED)
        assert bool((big == 3.0).all())
    release()


def test_plan_of_other_sizes():
    """A plan of more ids, or of a larger table, in the same workspace: the
    apply of the smaller sizes finds a stamp that is not its own."""
    n1, n2, rows1, rows2 = 30_000, 12_000, 90_000, 40_000
    size = E.engram_scatter_add_workspace(n1, rows1, DIM, E.SCATTER_ROWSPARSE)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    ids = _ids(n1, rows1, 5)
    grads = workloads.make_grads(n1, DIM, 6, "cuda")
    E.engram_scatter_plan(ids, rows1, DIM, workspace=ws)
    uid, val, u, err = _apply_sparse(grads[:n2], ws, rows1, n2)     # other n
    assert u == 0 and err == E.ERR_NO_PLAN and _untouched(uid, val)
    uid, val, u, err = _apply_sparse(grads, ws, rows2, n1)          # other table_rows
    assert u == 0 and err == E.ERR_NO_PLAN and _untouched(uid, val)
    big = torch.full((rows1, DIM), 3.0, dtype=torch.float32, device="cuda")
    derr = torch.zeros(1, dtype=torch.int64, device="cuda")
    E.engram_scatter_apply(grads, ws, rows2, grad_table=big[:rows2], err_count=derr)
    torch.cuda.synchronize()
    assert int(derr.item()) == E.ERR_NO_PLAN and bool((big == 3.0).all())
    # the plan's own sizes: the sums of the one-call form, and no error
    uid, val, u, err = _apply_sparse(grads, ws, rows1, n1)
    want_uid, want_val, want_cnt = E.engram_scatter_add_rowsparse(ids, grads, rows1)
    torch.cuda.synchronize()
    assert err == 0 and u == int(want_cnt.item()) > 0
    assert torch.equal(uid[:u], want_uid[:u])
    assert torch.equal(val[:u].view(torch.int32), want_val[:u].view(torch.int32))
    assert bool((uid[n1:] == -7).all())
    release()


def test_stalled_plan_is_refused():
    """A plan whose wait expired is marked in the workspace; the mark is set
    here from the host (the plan's scalars start the workspace: U, then the
    stall flag, then the stamp), as no kernel is made to stall."""
    n, rows = 25_000, 60_000
    size = E.engram_scatter_add_workspace(n, rows, DIM, E.SCATTER_ROWSPARSE)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    ids = _ids(n, rows, 8)
    grads = workloads.make_grads(n, DIM, 9, "cuda")
    E.engram_scatter_plan(ids, rows, DIM, workspace=ws)
    torch.cuda.synchronize()
    stamp = ws[:24].view(torch.int64).cpu().numpy()
    assert stamp[1] == n and stamp[2] == rows          # where the stamp lives
    ws[4:8] = torch.tensor([1, 0, 0, 0], dtype=torch.uint8, device="cuda")
    uid, val, u, err = _apply_sparse(grads, ws, rows, n)
    assert u == 0 and err == E.ERR_STALLED and _untouched(uid, val)
    ws[4:8] = 0
    uid, val, u, err = _apply_sparse(grads, ws, rows, n)
    assert err == 0 and u > 0
    release()
