"""Parity at full size: the 200M x 256 bf16 table (102.4 GB) resident in HBM.

Row ids are compared with the oracle in full.  Gathered rows are compared
with the oracle on a sample of outputs (the oracle gathers from a host copy
of just the table rows those outputs need) and, over every output, with
torch's index_select on the device.  The e2e backward (row-sparse) is
compared with the oracle in full.  These use the calls the benchmark times.
"""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, host_f32, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

SAMPLE = 8192


def sampled_gather_check(oracle, rows_host, out, table, seed):
    dim = table.shape[1]
    flat_rows = rows_host.reshape(-1)
    pick = np.random.Generator(np.random.PCG64(seed)).choice(flat_rows.size, SAMPLE,
                                                            replace=False)
    uniq, local = np.unique(flat_rows[pick], return_inverse=True)
    small_table = bits(table.index_select(0, dev(uniq)))
    want, bad = oracle.gather(local.astype(np.int64), small_table)
    assert bad == 0
    got = bits(out.view(-1, dim).index_select(0, dev(pick.astype(np.int64))))
    assert np.array_equal(got, want)
    # every output row against torch's index_select on the device
    assert torch.equal(out.view(-1, dim), table.index_select(0, dev(flat_rows)))


def forward(wl, tok, seg, table, mult):
    rows = E.engram_hash(dev(tok), wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
                         wl.primes, wl.offsets, wl.table_rows,
                         seq_ids=None if seg is None else dev(seg))
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = E.engram_gather(rows, table, err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return rows, out


def test_full_scale_forward(oracle):
    wl = workloads.full()
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    mult = wl.multipliers()
    tok, seg = wl.tokens(0, with_segments=True)
    for s in (None, seg):
        rows, out = forward(wl, tok, s, table, mult)
        want = oracle.hash(tok, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
                           wl.primes, wl.offsets, s)
        rows_host = rows.cpu().numpy()
        assert np.array_equal(rows_host, want)
        assert out.shape == (1, 32768, 32, 256)
        sampled_gather_check(oracle, rows_host, out, table, wl.seed)
        del rows, out
    # the 8-way context-parallel split: each slice's forward reads its history
    # across the boundary and equals the same slice of the whole forward
    step = tok.shape[1] // 8
    for r in range(8):
        a, b = r * step, (r + 1) * step
        sl = E.forward_global_slice(dev(tok), a, b, table, wl.ngram_size, wl.heads_per_ngram,
                                    wl.eos_id, mult, wl.primes, wl.offsets, seq_ids=dev(seg))
        torch.cuda.synchronize()
        want = oracle.hash_global_slice(tok, a, b, wl.ngram_size, wl.heads_per_ngram,
                                        wl.eos_id, mult, wl.primes, wl.offsets, seg)
        assert sl.shape == (1, step, 32 * 256)
        sampled_gather_check(oracle, want, sl.view(1, step, 32, 256), table, wl.seed + r)
        del sl
    del table
    release()


def test_e2e_forward_backward(oracle):
    wl = workloads.e2e()
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    mult = wl.multipliers()
    tok = wl.tokens(0)
    rows, out = forward(wl, tok, None, table, mult)
    want = oracle.hash(tok, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes,
                       wl.offsets)
    rows_host = rows.cpu().numpy()
    assert np.array_equal(rows_host, want)
    sampled_gather_check(oracle, rows_host, out, table, wl.seed + 1)
    # the fused forward the benchmark times gives the same rows and values
    fused_ids = torch.empty_like(rows)
    fused = E.engram_lookup(dev(tok), table, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
                            wl.primes, wl.offsets, row_ids=fused_ids)
    torch.cuda.synchronize()
    assert torch.equal(fused_ids, rows)
    assert torch.equal(fused.view(-1), out.view(-1))
    del out, fused, table
    release()

    grads = workloads.make_grads(wl.lookups, wl.dim, wl.seed + 2, "cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    uid, uval, count = E.engram_scatter_add_rowsparse(rows.view(-1), grads, wl.table_rows,
                                                      err_count=err)
    # the plan the benchmark times (from the tokens) gives the same output
    perr = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws_t = E.engram_scatter_plan_tokens(dev(tok), wl.table_rows, wl.dim, wl.ngram_size,
                                        wl.heads_per_ngram, wl.eos_id, mult, wl.primes,
                                        wl.offsets, err_count=perr)
    uid_t, uval_t, count_t = E.engram_scatter_apply(grads, ws_t, wl.table_rows, err_count=perr)
    torch.cuda.synchronize()
    assert int(perr.item()) == 0
    ut = int(count_t.item())
    assert ut == int(count.item())
    assert torch.equal(uid_t[:ut], uid[:ut])
    assert torch.equal(uval_t[:ut].view(torch.int32), uval[:ut].view(torch.int32))
    del uid_t, uval_t, ws_t
    u = int(count.item())
    assert int(err.item()) == 0
    want_uid, want_val, bad = oracle.scatter_add_rowsparse(rows_host.reshape(-1), bits(grads),
                                                           wl.dim, wl.table_rows)
    assert bad == 0 and u == want_uid.size
    assert 0.5 * wl.lookups < u < wl.lookups
    assert np.array_equal(uid[:u].cpu().numpy(), want_uid)
    assert np.array_equal(host_f32(uval[:u]).view(np.uint32), want_val.view(np.uint32))
    del uid, uval
    release()

    # the backward fused with one SignSGD step on the 102.4 GB table: every
    # touched row against the oracle's step on a host copy of those rows
    lr = 2.0 ** -6
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    touched = dev(want_uid)
    before = bits(table.index_select(0, touched))
    want_rows, bad = oracle.signsgd_rowsparse(np.arange(u, dtype=np.int64), want_val, before, lr)
    assert bad == 0
    ws = E.engram_scatter_plan(rows.view(-1), wl.table_rows, wl.dim)
    E.engram_scatter_apply_signsgd(grads, ws, table, lr)
    torch.cuda.synchronize()
    assert np.array_equal(bits(table.index_select(0, touched)), want_rows)
    assert not np.array_equal(want_rows, before)
    del grads, table, ws
    release()


def test_e2e_pad_tail_backward(oracle):
    """The e2e shape on packs whose row tails are pad tokens in a segment of
    their own: every head hashes the tail into one row, runs of thousands of
    terms that the apply sums in chunks of 512 sorted positions.  The fused forward's ids, the plan
    made from the tokens and its row-sparse apply, and the SignSGD apply, all
    at full size against the oracle (the backward in full)."""
    wl = workloads.e2e_padtail()
    mult = wl.multipliers()
    tok, seg = wl.tokens(0, with_segments=True)
    args = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes, wl.offsets)
    want_rows = oracle.hash(tok, *args, seg)
    flat = want_rows.reshape(-1)
    counts = np.unique(flat, return_counts=True)[1]
    assert counts.max() > 4 * 512      # the tail's rows cross several chunks each
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    ids = torch.empty((tok.shape[0], tok.shape[1], wl.heads), dtype=torch.int64, device="cuda")
    out = E.engram_lookup(dev(tok), table, *args, seq_ids=dev(seg), row_ids=ids)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), want_rows)
    sampled_gather_check(oracle, want_rows, out, table, wl.seed)
    del out, ids
    release()
    grads = workloads.make_grads(wl.lookups, wl.dim, wl.seed + 2, "cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = E.engram_scatter_plan_tokens(dev(tok), wl.table_rows, wl.dim, *args, seq_ids=dev(seg),
                                      err_count=err)
    uid, uval, cnt = E.engram_scatter_apply(grads, ws, wl.table_rows, err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want_uid, want_val, bad = oracle.scatter_add_rowsparse(flat, bits(grads), wl.dim,
                                                           wl.table_rows)
    u = int(cnt.item())
    assert bad == 0 and u == want_uid.size
    assert np.array_equal(uid[:u].cpu().numpy(), want_uid)
    assert np.array_equal(host_f32(uval[:u]).view(np.uint32), want_val.view(np.uint32))
    del uid, uval
    # the same plan fused with one SignSGD step: every touched row
    lr = 2.0 ** -6
    touched = dev(want_uid)
    before = bits(table.index_select(0, touched))
    want_t, bad = oracle.signsgd_rowsparse(np.arange(u, dtype=np.int64), want_val, before, lr)
    E.engram_scatter_apply_signsgd(grads, ws, table, lr, err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(bits(table.index_select(0, touched)), want_t)
    del grads, table, ws
    release()


def test_many_chunk_crossing_runs(oracle):
    """48,000 long runs, each crossing a boundary of the apply's 512-position
    chunks, over more chunks (about 66,000) than the apply's second launch
    reads in one round: every distinct row id in full, and the sums of a
    sample of rows against the oracle (a row's sum depends on its own
    positions only, so the oracle sums just those)."""
    rng = np.random.Generator(np.random.PCG64(4242))
    rows, dim, n_runs = 1 << 24, 8, 48_000
    lens = rng.integers(520, 900, size=n_runs)
    keys = rng.permutation(rows)[:n_runs].astype(np.int64)
    ids = rng.permutation(np.repeat(keys, lens))
    assert ids.size > 256 * 256 * 512
    grads = workloads.make_grads(ids.size, dim, 4243, "cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = E.engram_scatter_plan(dev(ids), rows, dim, err_count=err)
    uid, uval, cnt = E.engram_scatter_apply(grads, ws, rows, err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    want_uid = np.sort(keys)
    u = int(cnt.item())
    assert u == n_runs
    assert np.array_equal(uid[:u].cpu().numpy(), want_uid)
    picked = np.sort(rng.choice(want_uid, 512, replace=False))
    where = np.nonzero(np.isin(ids, picked))[0]
    sub_grads = bits(grads.index_select(0, dev(where.astype(np.int64))))
    w_uid, w_val, bad = oracle.scatter_add_rowsparse(ids[where], sub_grads, dim, rows)
    assert bad == 0 and np.array_equal(w_uid, picked)
    got = host_f32(uval.index_select(0, dev(np.searchsorted(want_uid, picked).astype(np.int64))))
    assert np.array_equal(got.view(np.uint32), w_val.view(np.uint32))
    del grads, ws, uid, uval
    release()
