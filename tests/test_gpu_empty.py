"""Empty inputs through the entry points of the path that take a batch: no
tokens (an empty batch, or rows of no positions) for the fused lookup and the
plan from the tokens; no lookups for the plan of ids, both forms of the
apply, the fused SignSGD apply and the allocation-free scatter-add; no
positions for the PLE convolution; an empty operation list.  Each call
succeeds, leaves every table it may write bit for bit as it was, and
reports zero distinct rows where it has a count."""
import pytest
import torch

from tests.gpu_helpers import needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

# ngram_size 3, two heads per order: four heads on disjoint row ranges
HARGS = (3, 2, 0, [1, 2, 3], [5, 7, 11, 13], [0, 5, 12, 23])
ROWS, DIM = 36, 16


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("shape", [(0, 16), (2, 0)])
def test_empty_token_batch(shape):
    tok = torch.zeros(shape, dtype=torch.int64, device="cuda")
    table = torch.randn((ROWS, DIM), device="cuda").to(torch.bfloat16)
    table0 = table.clone()
    err = torch.zeros(1, dtype=torch.int64, device="cuda")

    out = E.engram_lookup(tok, table, *HARGS)
    assert out.shape == (*shape, 4, DIM)
    rid = torch.empty((*shape, 4), dtype=torch.int64, device="cuda")
    E.engram_lookup(tok, table, *HARGS, out=out, row_ids=rid)

    ws = E.engram_scatter_plan_tokens(tok, ROWS, DIM, *HARGS, err_count=err)
    grads = torch.zeros((0, DIM), dtype=torch.bfloat16, device="cuda")
    count = torch.full((1,), 9, dtype=torch.int64, device="cuda")
    E.engram_scatter_apply(grads, ws, ROWS, num_unique=count, err_count=err)
    gtab = torch.ones((ROWS, DIM), dtype=torch.float32, device="cuda")
    E.engram_scatter_apply(grads, ws, ROWS, grad_table=gtab, err_count=err)
    E.engram_scatter_apply_signsgd(grads, ws, table, 2.0 ** -4, err_count=err)
    torch.cuda.synchronize()
    assert int(count.item()) == 0
    assert torch.equal(gtab, torch.ones_like(gtab))
    assert torch.equal(_bits(table), _bits(table0))
    assert int(err.item()) == 0
    release()


def test_empty_ids_plan_apply_and_noalloc():
    ids = torch.zeros(0, dtype=torch.int64, device="cuda")
    grads = torch.zeros((0, DIM), dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = E.engram_scatter_plan(ids, ROWS, DIM, err_count=err)
    count = torch.full((1,), 9, dtype=torch.int64, device="cuda")
    E.engram_scatter_apply(grads, ws, ROWS, num_unique=count, err_count=err)
    torch.cuda.synchronize()
    assert int(count.item()) == 0

    uid = torch.full((1,), -5, dtype=torch.int64, device="cuda")
    uval = torch.full((1, DIM), 3.0, dtype=torch.float32, device="cuda")
    count.fill_(9)
    E.engram_scatter_add_rowsparse_noalloc(ids, grads, ROWS, uid, uval, count, err_count=err)
    torch.cuda.synchronize()
    assert int(count.item()) == 0
    assert int(uid.item()) == -5 and bool((uval == 3.0).all())  # nothing written past the count
    assert int(err.item()) == 0
    release()


@pytest.mark.parametrize("shape", [(0, 8, 16), (2, 0, 16)])
def test_empty_conv(shape):
    x = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    w = torch.randn((16, 4), device="cuda").to(torch.bfloat16)
    out = E.engram_ple_conv(x, w, 3)
    torch.cuda.synchronize()
    assert out.shape == shape


def test_empty_schedule():
    E.Schedule().run()
