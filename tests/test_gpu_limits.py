"""The sorted scatter-add past 2^31 ids, near the largest input it takes
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
the host.  About 100 GB of device memory."""
import numpy as np
import pytest
import torch

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
