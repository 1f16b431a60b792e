"""The path captured in HIP graphs and replayed: the plan from the tokens,
the fused forward and the apply (row-sparse and dense), as the benchmark's
graph schedule runs them.  Each graph is replayed several times, with other
work launched call by call and synchronizations between the replays, and
every replay is compared bit for bit with the same calls launched one by one
(which the other tests compare with the oracle); one replay's row-sparse
result is also compared with the oracle directly."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, host_f32, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")


def _setup():
    wl = workloads.backward()
    hargs = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, wl.multipliers(), wl.primes,
             wl.offsets)
    toks = [dev(wl.tokens(k)) for k in range(2)]
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    grads = workloads.make_grads(wl.lookups, wl.dim, wl.seed + 2, "cuda")
    return wl, hargs, toks, table, grads


def _rowsparse_outputs(wl):
    R, D = wl.lookups, wl.dim
    return (torch.empty(R, dtype=torch.int64, device="cuda"),
            torch.empty((R, D), dtype=torch.float32, device="cuda"),
            torch.zeros(1, dtype=torch.int64, device="cuda"))


def test_graph_replays_match_calls(oracle):
    wl, hargs, toks, table, grads = _setup()
    R, D = wl.lookups, wl.dim
    mode = E.SCATTER_ROWSPARSE
    ws = torch.empty(E.engram_scatter_add_workspace(R, wl.table_rows, D, mode),
                     dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")

    # the calls one by one, per batch: the reference
    want = []
    for t in toks:
        out = E.engram_lookup(t, table, *hargs)
        E.engram_scatter_plan_tokens(t, wl.table_rows, D, *hargs, workspace=ws, err_count=err)
        uid, uval, cnt = E.engram_scatter_apply(grads, ws, wl.table_rows, err_count=err)
        torch.cuda.synchronize()
        u = int(cnt.item())
        want.append((out.clone(), u, uid[:u].clone(), uval[:u].clone()))
    assert int(err.item()) == 0

    # one graph per batch: plan on a branch, joined before the apply
    out = torch.empty((toks[0].shape[0], toks[0].shape[1], wl.heads, D), dtype=torch.bfloat16,
                      device="cuda")
    uid, uval, cnt = _rowsparse_outputs(wl)
    side = torch.cuda.Stream()
    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    graphs = []
    for t in toks:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                E.engram_scatter_plan_tokens(t, wl.table_rows, D, *hargs, workspace=ws,
                                             err_count=err, stream=side)
            E.engram_lookup(t, table, *hargs, out=out)
            cur.wait_stream(side)
            E.engram_scatter_apply(grads, ws, wl.table_rows, unique_ids=uid, unique_grads=uval,
                                   num_unique=cnt, err_count=err)
        graphs.append(g)
    torch.cuda.synchronize()

    other = torch.empty_like(ws)
    for rep in range(3):
        for b, g in enumerate(graphs):
            uval.zero_()
            cnt.zero_()
            g.replay()
            torch.cuda.synchronize()
            w_out, w_u, w_uid, w_uval = want[b]
            u = int(cnt.item())
            assert u == w_u, (rep, b)
            assert torch.equal(out.view(torch.int16), w_out.view(torch.int16)), (rep, b)
            assert torch.equal(uid[:u], w_uid), (rep, b)
            assert torch.equal(uval[:u].view(torch.int32), w_uval.view(torch.int32)), (rep, b)
            # other work launched call by call between the replays
            E.engram_scatter_plan_tokens(toks[1 - b], wl.table_rows, D, *hargs,
                                         workspace=other, err_count=err)
            E.engram_scatter_apply(grads, other, wl.table_rows, err_count=err)
            torch.cuda.synchronize()
    assert int(err.item()) == 0

    # the last replay's batch against the oracle
    rows = oracle.hash(toks[1].cpu().numpy(), *hargs).reshape(-1)
    o_uid, o_val, bad = oracle.scatter_add_rowsparse(rows, bits(grads), D, wl.table_rows)
    u = int(cnt.item())
    assert bad == 0 and u == o_uid.size
    assert np.array_equal(uid[:u].cpu().numpy(), o_uid)
    assert np.array_equal(host_f32(uval[:u]).view(np.uint32), o_val.view(np.uint32))
    del graphs, table, grads, ws, other
    release()


def test_graph_replays_dense():
    """The dense apply in a graph, replayed onto a cleared gradient table:
    every replay equals the apply launched on its own."""
    wl, hargs, toks, table, grads = _setup()
    R, D = wl.lookups, wl.dim
    ws = torch.empty(E.engram_scatter_add_workspace(R, wl.table_rows, D, E.SCATTER_SORTED),
                     dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    gtab = workloads.make_grad_table(wl.table_rows, D, None, "cuda")
    E.engram_scatter_plan_tokens(toks[0], wl.table_rows, D, *hargs, workspace=ws, err_count=err)
    E.engram_scatter_apply(grads, ws, wl.table_rows, grad_table=gtab, err_count=err)
    torch.cuda.synchronize()
    ref_rows = dev(np.unique(E.engram_hash(toks[0], *hargs, wl.table_rows).cpu().numpy()))
    want = gtab.index_select(0, ref_rows).clone()

    cap = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        E.engram_scatter_plan_tokens(toks[0], wl.table_rows, D, *hargs, workspace=ws,
                                     err_count=err)
        E.engram_scatter_apply(grads, ws, wl.table_rows, grad_table=gtab, err_count=err)
    torch.cuda.synchronize()
    for rep in range(3):
        gtab.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = gtab.index_select(0, ref_rows)
        assert torch.equal(got.view(torch.int32), want.view(torch.int32)), rep
        # nothing else touched
        assert not bool(gtab.index_fill_(0, ref_rows, 0.0).any()), rep
        E.engram_scatter_plan_tokens(toks[1], wl.table_rows, D, *hargs, workspace=ws,
                                     err_count=err)
        torch.cuda.synchronize()
    assert int(err.item()) == 0
    del g, gtab, table, grads, ws
    release()
