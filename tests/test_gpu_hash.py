"""GPU parity of engram_hash against the oracle: bit-exact row ids."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import dev, needs_gpu
from tests.test_oracle_hash import EDGE, P61, P63, WINDOW_CASES

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")


def gpu_rows(tok, n, J, eos, mult, primes, offs, rows, seg=None):
    out = E.engram_hash(dev(tok), n, J, eos, mult, primes, offs, rows,
                        seq_ids=None if seg is None else dev(seg))
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("name", ["tiny", "medium", "full", "backward", "e2e"])
@pytest.mark.parametrize("segments", [False, True])
def test_workload_rows_match_oracle(oracle, name, segments):
    wl = workloads.get(name)
    tok, seg = wl.tokens(0, with_segments=True)
    if segments and seg is None:
        seg = workloads.random_segments(tok.shape, 300, wl.seed)
    if not segments:
        seg = None
    mult = wl.multipliers()
    want = oracle.hash(tok, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
                       wl.primes, wl.offsets, seg)
    got = gpu_rows(tok, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes,
                   wl.offsets, wl.table_rows, seg)
    assert got.shape == want.shape
    assert np.array_equal(got, want)


def test_page_multipliers(oracle):
    wl = workloads.tiny()
    tok = wl.tokens(1)
    mult = workloads.PAGE_LAYER_MULTIPLIERS
    want = oracle.hash(tok, 3, 2, 0, mult, wl.primes, wl.offsets)
    got = gpu_rows(tok, 3, 2, 0, mult, wl.primes, wl.offsets, wl.table_rows)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: c["name"])
def test_golden_windows(oracle, case):
    """The hand-written window cases, with seeded full-range multipliers."""
    n, J = case["n"], 3
    tok = np.array([case["tokens"]], dtype=np.int64)
    seg = None if case["seg"] is None else np.array([case["seg"]], dtype=np.int64)
    primes = [1009, 1013, 1019] * (n - 1)
    offs = workloads.cumulative_offsets(primes)
    for variant in range(3):
        mult = workloads.seeded_multipliers(n, 500 + variant)
        want = oracle.hash(tok, n, J, case["eos"], mult, primes, offs, seg)
        got = gpu_rows(tok, n, J, case["eos"], mult, primes, offs, sum(primes), seg)
        assert np.array_equal(got, want), variant


@pytest.mark.parametrize("seed", range(4))
def test_int64_edges(oracle, seed):
    """Wrapping products and sums at the int64 edges; moduli from 1 to the
    largest prime below 2^63 (Barrett reduction's extremes)."""
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    n, J = 4, 3
    tok = np.array(rng.choice(EDGE, size=(5, 97)), dtype=np.int64)
    mult = np.array(rng.choice(EDGE + [-3, 23703573157769], size=n), dtype=np.int64)
    primes = [1, 2, 3, P61, P63, 2147483647, 4294967311, 97, (1 << 62) + 135]
    offs = [0] * 9
    seg = rng.integers(0, 2, size=tok.shape).cumsum(axis=1)
    for s in (None, seg):
        want = oracle.hash(tok, n, J, 248044, mult, primes, offs, s)
        got = gpu_rows(tok, n, J, 248044, mult, primes, offs, P63, s)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("shape,n,J", [((3, 77), 8, 8), ((1, 1), 3, 2), ((5, 1), 4, 2),
                                       ((2, 200), 2, 64), ((7, 65), 3, 1), ((1, 4097), 5, 4)])
def test_ragged_and_extreme_shapes(oracle, shape, n, J):
    rng = np.random.Generator(np.random.PCG64(sum(shape) + n * 13 + J))
    tok = rng.integers(0, 50, size=shape).astype(np.int64)   # eos 0 frequent
    H = (n - 1) * J
    primes = workloads.primes_above(1000, H)
    offs = workloads.cumulative_offsets(primes)
    mult = workloads.seeded_multipliers(n, 9)
    seg = workloads.random_segments(shape, 10, 3)
    for s in (None, seg):
        want = oracle.hash(tok, n, J, 0, mult, primes, offs, s)
        got = gpu_rows(tok, n, J, 0, mult, primes, offs, sum(primes), s)
        assert np.array_equal(got, want)


def test_empty_batch():
    tok = torch.zeros((0, 16), dtype=torch.int64, device="cuda")
    out = E.engram_hash(tok, 3, 2, 0, [1, 2, 3], [5, 7, 11, 13], [0, 5, 12, 23], 36)
    assert out.shape == (0, 16, 4)


def test_rejects_bad_constants_on_device_tensors():
    tok = torch.zeros((1, 8), dtype=torch.int64, device="cuda")
    with pytest.raises(E.EngramError):
        E.engram_hash(tok, 3, 2, 0, [1, 2, 3], [5, 7, 11, 13], [0, 5, 12, 30], 36)


def test_writes_into_caller_buffer_on_caller_stream(oracle):
    wl = workloads.tiny()
    tok = wl.tokens(2)
    mult = wl.multipliers()
    out = torch.full((2, 128, 4), -7, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    t = dev(tok)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        E.engram_hash(t, 3, 2, 0, mult, wl.primes, wl.offsets, wl.table_rows, out=out)
    side.synchronize()
    want = oracle.hash(tok, 3, 2, 0, mult, wl.primes, wl.offsets)
    assert np.array_equal(out.cpu().numpy(), want)
