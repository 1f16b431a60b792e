"""engram_run_ops through the binding's Schedule: steps built once and
enqueued with one native call each (the next batch's plan on a side stream
behind an event, the fused forward and the apply on the main stream) give
exactly what the same calls give one by one; a failing operation is
reported with its index, and the operations before it still run."""
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import dev, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

N_BATCHES = 4


def _setup(name="backward"):
    wl = workloads.get(name)
    hargs = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, wl.multipliers(), wl.primes,
             wl.offsets)
    toks = [dev(wl.tokens(k)) for k in range(N_BATCHES)]
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    grads = workloads.make_grads(wl.lookups, wl.dim, wl.seed + 2, "cuda")
    return wl, hargs, toks, table, grads


def test_scheduled_steps_match_calls():
    wl, hargs, toks, table, grads = _setup()
    R, D = wl.lookups, wl.dim
    need = E.engram_scatter_add_workspace(R, wl.table_rows, D, E.SCATTER_ROWSPARSE)
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda") for _ in range(2)]
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = torch.empty((toks[0].shape[0], toks[0].shape[1], wl.heads, D), dtype=torch.bfloat16,
                      device="cuda")
    uid = torch.empty(R, dtype=torch.int64, device="cuda")
    uval = torch.empty((R, D), dtype=torch.float32, device="cuda")
    cnt = torch.zeros(1, dtype=torch.int64, device="cuda")

    # the reference: every batch's calls one by one on one stream
    ref_ws = torch.empty_like(wss[0])
    want = []
    for t in toks:
        o = E.engram_lookup(t, table, *hargs)
        E.engram_scatter_plan_tokens(t, wl.table_rows, D, *hargs, workspace=ref_ws)
        u_, v_, c_ = E.engram_scatter_apply(grads, ref_ws, wl.table_rows)
        torch.cuda.synchronize()
        c = int(c_.item())
        want.append((o.clone(), c, u_[:c].clone(), v_[:c].clone()))

    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev_plan = [torch.cuda.Event() for _ in range(2)]
    ev_apply = [torch.cuda.Event() for _ in range(2)]
    scheds = []
    for k in range(N_BATCHES):
        nk = (k + 1) % N_BATCHES
        s = E.Schedule()
        s.wait(ev_apply[nk % 2], stream=side)
        s.plan_tokens(toks[nk], wl.table_rows, D, *hargs, workspace=wss[nk % 2], err_count=err,
                      stream=side)
        s.record(ev_plan[nk % 2], stream=side)
        s.lookup(toks[k], table, *hargs, out=out, stream=main)
        s.wait(ev_plan[k % 2], stream=main)
        s.apply(grads, wss[k % 2], wl.table_rows, unique_ids=uid, unique_grads=uval,
                num_unique=cnt, err_count=err, stream=main)
        s.record(ev_apply[k % 2], stream=main)
        assert len(s) == 7
        scheds.append(s)
    # batch 0's plan first, as the step before would have made it
    E.engram_scatter_plan_tokens(toks[0], wl.table_rows, D, *hargs, workspace=wss[0],
                                 err_count=err)
    ev_plan[0].record(main)
    for step in range(2 * N_BATCHES + 1):
        k = step % N_BATCHES
        uval.zero_()
        scheds[k].run()
        torch.cuda.synchronize()
        w_out, w_c, w_uid, w_uval = want[k]
        c = int(cnt.item())
        assert c == w_c, step
        assert torch.equal(out.view(torch.int16), w_out.view(torch.int16)), step
        assert torch.equal(uid[:c], w_uid), step
        assert torch.equal(uval[:c].view(torch.int32), w_uval.view(torch.int32)), step
    assert int(err.item()) == 0
    del scheds
    release()


def test_scheduled_signsgd_matches_call():
    wl, hargs, toks, table, grads = _setup()
    R, D = wl.lookups, wl.dim
    ws = E.engram_scatter_plan_tokens(toks[0], wl.table_rows, D, *hargs)
    a, b = table.clone(), table.clone()
    lr = 2.0 ** -6
    E.engram_scatter_apply_signsgd(grads, ws, a, lr)
    E.Schedule().apply_signsgd(grads, ws, b, lr).run()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert not torch.equal(a.view(torch.int16), table.view(torch.int16))
    del a, b, ws
    release()


def test_failing_operation_reports_its_index():
    wl, hargs, toks, table, grads = _setup()
    D = wl.dim
    out = torch.zeros((toks[0].shape[0], toks[0].shape[1], wl.heads, D), dtype=torch.bfloat16,
                      device="cuda")
    small = torch.empty(16, dtype=torch.uint8, device="cuda")  # far too small a workspace
    s = E.Schedule()
    s.lookup(toks[0], table, *hargs, out=out)
    s.plan_tokens(toks[0], wl.table_rows, D, *hargs, workspace=small)
    with pytest.raises(E.EngramError) as exc:
        s.run()
    assert exc.value.status == E.ENGRAM_EWORKSPACE
    assert "operation 1" in str(exc.value)
    torch.cuda.synchronize()
    want = E.engram_lookup(toks[0], table, *hargs)
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))  # op 0 ran
    release()
