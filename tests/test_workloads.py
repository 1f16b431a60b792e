"""The seeded input generators: shapes, determinism, and the stated recipes."""
import numpy as np
import pytest

from gram_hashed_embedding_amd import workloads as W


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_tokens_deterministic_and_shaped(name):
    wl = W.get(name)
    a = wl.tokens(0)
    b = wl.tokens(0)
    c = wl.tokens(1)
    assert a.shape == (wl.batch, wl.seq) and a.dtype == np.int64
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert a.min() >= 0 and a.max() < W.VOCAB


def test_table_shapes_and_primes():
    assert W.tiny().table_rows == 4062 and W.tiny().offsets == (0, 1009, 2022, 3041)
    med = W.medium()
    assert med.primes[0] == 1048583 and med.primes[-1] == 1048793
    assert med.table_rows == 16_778_782
    full = W.full()
    assert len(full.primes) == 32 and full.primes[-1] == 6249989
    assert sum(full.primes) == 199_994_628 and full.table_rows == 200_000_000
    e2e = W.e2e()
    assert len(e2e.primes) == 24 and e2e.primes[0] == 8332913
    assert sum(e2e.primes) == 199_995_086 and e2e.table_rows == 200_000_000
    for wl in (W.tiny(), med, full, W.backward(), e2e):
        assert all(W.is_prime(p) for p in wl.primes)
        assert wl.offsets[-1] + wl.primes[-1] <= wl.table_rows


def test_lookup_counts():
    assert W.tiny().lookups == 1024
    assert W.medium().lookups == 262_144
    assert W.full().lookups == 1_048_576
    assert W.backward().lookups == 262_144
    assert W.e2e().lookups == 1_572_864


def test_packed_documents_end_with_eos():
    wl = W.full()
    tok, seg = wl.tokens(0, with_segments=True)
    assert seg is not None and seg[0, 0] == 0
    ends = np.nonzero(np.diff(seg[0]))[0]          # last position of each doc
    assert (tok[0, ends] == W.EOS_ID).all()
    lens = np.diff(np.concatenate([[-1], ends]))
    assert 300 < lens.mean() < 8000


def test_zipf_is_skewed():
    tok = W.zipf_tokens(np.random.Generator(np.random.PCG64(0)), (200_000,), 1.1)
    counts = np.bincount(tok)
    assert counts[1] > counts[10] > counts[1000]
    assert tok.min() >= 1


def test_multipliers_odd_full_range():
    m = W.seeded_multipliers(4, 5)
    assert (m % 2 != 0).all()
    assert np.abs(m).max() > 1 << 40
