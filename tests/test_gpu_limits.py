"""Inputs past 2^31 lookups.

The sorted scatter-add near the largest input it takes
(n < 2^32 - 1: its plan keeps 32-bit sorted keys, flat indices, positions
and slots).  N = 2^31 + 2^20 + 123 ids into a table of M = 1,000,003 rows:
id i is row i mod M, so every row holds about 2,150 positions spread over
the whole index range, those past 2^31 included, and its run spans several
512-position chunks of the sorted order (the split-run path and the
apply's second launch).  Gradient element e of id i is the 3-bit field of
i at a shift of its own (up to bit 31), as a bf16 integer: every sum is an
exact integer in fp32, so a position given to the wrong row, dropped or
counted twice changes a result.  Checked: the dense table's column totals
against fp64 totals of the gradients (torch on the device), and 512
sampled rows (the first, the last, and the row of position 2^31 among
them) against the oracle, which sums each row's gradient rows copied to
the host.  About 100 GB of device memory.

The forward (hash and fused lookup) over one row of 2^30 + 77 tokens with
two heads (a bigram and a trigram head): 2^31 + 154 lookups, and a hash
grid the kernel covers by striding (64 tokens of 256 threads a block would
take more than 2^32 - 1 threads in one launch).  Every output
row is compared with torch's index_select of the hashed ids, and the ids
and output rows of 4,096 sampled positions (the first, the last, and those
on both sides of lookup index 2^31 among them) with the oracle, which
hashes each sampled position's window of tokens and gathers from a host
copy of the rows it names.  About 60 GB of device memory."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, host_f32, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

N = (1 << 31) + (1 << 20) + 123
M = 1_000_003
D = 8
SHIFTS = (0, 3, 6, 9, 14, 20, 26, 29)
CHUNK = 1 << 26


def test_sorted_scatter_past_2_31_ids(oracle):
    ids = torch.empty(N, dtype=torch.int64, device="cuda")
    grads = torch.empty((N, D), dtype=torch.bfloat16, device="cuda")
    want_total = torch.zeros(D, dtype=torch.int64, device="cuda")
    for c0 in range(0, N, CHUNK):
        i = torch.arange(c0, min(c0 + CHUNK, N), dtype=torch.int64, device="cuda")
        ids[c0:c0 + i.numel()] = i % M
        g = torch.stack([(i >> s) & 7 for s in SHIFTS], dim=1)
        grads[c0:c0 + i.numel()] = g.to(torch.bfloat16)
        want_total += g.sum(0)
        del i, g
    gtab = torch.zeros((M, D), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    print(f"scatter-add of {N} ids into {M} rows", flush=True)
    E.engram_scatter_add(ids, grads, gtab, err_count=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # every position lands exactly once: column totals (exact integers in fp64)
    assert torch.equal(gtab.double().sum(0), want_total.double())

    rng = np.random.Generator(np.random.PCG64(31))
    rows = np.unique(np.concatenate([np.array([0, 1, M - 1, (N - 1) % M, (1 << 31) % M]),
                                     rng.choice(M, 507, replace=False)]))
    counts = (N - 1 - rows) // M + 1
    pos = np.concatenate([r + M * np.arange(k, dtype=np.int64) for r, k in zip(rows, counts)])
    pos_d = dev(pos)
    assert np.array_equal(ids.index_select(0, pos_d).cpu().numpy(), np.repeat(rows, counts))
    local = np.repeat(np.arange(rows.size, dtype=np.int64), counts)
    want, bad = oracle.scatter_add_dense(local, bits(grads.index_select(0, pos_d)),
                                         np.zeros((rows.size, D), dtype=np.float32))
    assert bad == 0
    got = host_f32(gtab.index_select(0, dev(rows)))
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    del ids, grads, gtab, pos_d
    release()


T = (1 << 30) + 77  # tokens of the forward: two heads, 2^31 + 154 lookups
COMPARE = 1 << 24   # output rows per index_select comparison


def test_forward_past_2_31_lookups(oracle):
    n, J, eos = 3, 1, 0
    mult = [3, 1_000_003, 7919 * 65537]
    primes, offs = [999_983, 1_000_003], [0, 999_983]
    hargs = (n, J, eos, mult, primes, offs)
    rows_total = sum(primes)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(2031)
    tok = torch.randint(0, 50_000, (1, T), generator=gen, device="cuda", dtype=torch.int64)
    table = workloads.make_table(rows_total, D, 2031, "cuda")
    print(f"lookup of {T} tokens x 2 heads", flush=True)
    out = E.engram_lookup(tok, table, *hargs)
    ids = E.engram_hash(tok, *hargs, rows_total)
    torch.cuda.synchronize()
    flat_ids, flat_out = ids.view(-1), out.view(-1, D)
    for c0 in range(0, flat_ids.numel(), COMPARE):
        c1 = min(c0 + COMPARE, flat_ids.numel())
        want = table.index_select(0, flat_ids[c0:c1])
        assert torch.equal(flat_out[c0:c1].view(torch.int16), want.view(torch.int16)), c0
        del want

    rng = np.random.Generator(np.random.PCG64(2031))
    ts = np.unique(np.concatenate([np.array([0, 1, 2, (1 << 30) - 1, 1 << 30, T - 1]),
                                   rng.choice(T, 4090, replace=False)]))
    # the oracle's rows of each sampled position, from the n tokens ending there
    # (the history reaches n - 1 tokens back; positions 0 and 1 from the row's start)
    tok_row = tok[0]
    want_ids = np.empty((ts.size, 2), dtype=np.int64)
    for k, t in enumerate(ts[ts < n - 1]):
        want_ids[k] = oracle.hash(tok_row[:t + 1].cpu().numpy()[None], *hargs)[0, -1]
    late = ts >= n - 1
    win = dev(ts[late][:, None] + np.arange(-(n - 1), 1))
    windows = tok_row.index_select(0, win.view(-1)).view(-1, n).cpu().numpy()
    want_ids[late] = oracle.hash(windows, *hargs)[:, -1]
    ts_d = dev(ts)
    assert np.array_equal(ids[0].index_select(0, ts_d).cpu().numpy(), want_ids)
    uniq, local = np.unique(want_ids.reshape(-1), return_inverse=True)
    small_table = bits(table.index_select(0, dev(uniq)))
    want_rows, bad = oracle.gather(local.astype(np.int64), small_table)
    assert bad == 0
    got = bits(out[0].index_select(0, ts_d).reshape(-1, D))
    assert np.array_equal(got, want_rows)
    del tok, table, out, ids, flat_ids, flat_out
    release()
