"""GPU parity of engram_gather against the oracle: bit-exact bf16 rows."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")


@pytest.mark.parametrize("name", ["tiny", "medium"])
def test_forward_matches_oracle(oracle, name):
    """Hash then gather on the workload; the oracle gathers the oracle's own
    row ids from a host copy of the same table."""
    wl = workloads.get(name)
    tok = wl.tokens(0)
    mult = wl.multipliers()
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    rows = E.engram_hash(dev(tok), wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
                         wl.primes, wl.offsets, wl.table_rows)
    out = E.engram_gather(rows, table)
    got = bits(out).reshape(-1, wl.dim)
    want_rows = oracle.hash(tok, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
                            wl.primes, wl.offsets)
    want, bad = oracle.gather(want_rows.reshape(-1), bits(table))
    assert bad == 0
    assert out.shape == (wl.batch, wl.seq, wl.heads, wl.dim)
    assert np.array_equal(got, want)
    del table, out
    release()


@pytest.mark.parametrize("dim", [8, 16, 24, 40, 64, 128, 256, 512, 1024, 2048])
@pytest.mark.parametrize("n", [1, 7, 1000, 4099])
def test_dims_and_ragged_counts(oracle, dim, n):
    rng = np.random.Generator(np.random.PCG64(dim * 10007 + n))
    rows = 3001
    table = workloads.make_table(rows, dim, dim + n, "cuda", std=1.0)
    ids = rng.integers(0, rows, size=n).astype(np.int64)
    out = E.engram_gather(dev(ids), table)
    want, _ = oracle.gather(ids, bits(table))
    assert np.array_equal(bits(out).reshape(n, dim), want)


def test_padding_and_invalid_ids(oracle):
    table = workloads.make_table(100, 64, 5, "cuda", std=1.0)
    ids = np.array([3, -1, 99, 100, -2, 7, 1 << 40, -1, 0, -(1 << 62)], dtype=np.int64)
    ids = np.tile(ids, 37)
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    out = E.engram_gather(dev(ids), table, err_count=err)
    want, bad = oracle.gather(ids, bits(table))
    assert np.array_equal(bits(out).reshape(ids.size, 64), want)
    assert int(err.item()) == bad == 4 * 37


def test_empty():
    table = workloads.make_table(10, 32, 1, "cuda")
    out = E.engram_gather(torch.zeros(0, dtype=torch.int64, device="cuda"), table)
    assert out.shape == (0, 32)


def test_output_shape_follows_ids():
    table = workloads.make_table(50, 16, 1, "cuda")
    ids = torch.randint(0, 50, (2, 3, 4), device="cuda")
    out = E.engram_gather(ids, table)
    assert out.shape == (2, 3, 4, 16)
    assert torch.equal(out, table[ids])
