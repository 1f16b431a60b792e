"""CPU pins for the oracle's global-slice hash (no GPU, no HIP code).

Source: NeMo AutoModel v0.7 API page (qwen3_8_flash_next.engram),
Qwen3_8_FlashNextNGramEmbedding._forward_global_slice: the complete
replicated sequence is hashed, so a context-parallel slice keeps the raw
tokens before its first position and the EOS resets at the boundary; only
the slice is looked up.
"""
import numpy as np
import pytest

from gram_hashed_embedding_amd import workloads
from tests.test_oracle_hash import P61, WINDOW_CASES

SLICE_CASES = [c for c in WINDOW_CASES if c["slice"] is not None]


def test_slice_cases_present():
    assert len(SLICE_CASES) >= 2


def _unit_rows(oracle, case, k, start, end, whole_tokens=True):
    n, J = case["n"], 1
    H = n - 1
    primes = [P61] * H
    offsets = [1000 * (h + 1) for h in range(H)]
    mult = np.zeros(n, dtype=np.int64)
    mult[k] = 1
    tok = np.array([case["tokens"]], dtype=np.int64)
    seg = None if case["seg"] is None else np.array([case["seg"]], dtype=np.int64)
    if whole_tokens:
        rows = oracle.hash_global_slice(tok, start, end, n, J, case["eos"], mult, primes,
                                        offsets, seg)[0]
    else:  # the slice hashed as if it were a row of its own
        rows = oracle.hash(tok[:, start:end], n, J, case["eos"], mult, primes, offsets,
                           None if seg is None else seg[:, start:end])[0]
    return rows - np.array(offsets)


@pytest.mark.parametrize("case", SLICE_CASES, ids=lambda c: c["name"])
def test_slice_reads_history_across_the_boundary(oracle, case):
    """Unit multipliers expose the token k back: the slice must read the
    hand-written whole-row windows unchanged, at its first positions too."""
    start, end = case["slice"]
    for k in range(1, case["n"]):
        got = _unit_rows(oracle, case, k, start, end)
        for h in range(case["n"] - 1):
            want = case["expected"][k][start:end] if h + 2 > k else [0] * (end - start)
            assert list(got[:, h]) == want, (case["name"], k, h)


def test_slice_alone_would_lose_the_history(oracle):
    """Hashing the slice's tokens as a fresh row reads FILL at its first
    positions; the global slice does not (the reason the pages hash the
    replicated sequence)."""
    case = next(c for c in SLICE_CASES if c["name"] == "cp_slice_keeps_history")
    start, end = case["slice"]
    glob = _unit_rows(oracle, case, 1, start, end)
    alone = _unit_rows(oracle, case, 1, start, end, whole_tokens=False)
    assert list(glob[:, 0]) == [3, 4, 5]
    assert list(alone[:, 0]) == [0, 4, 5]


def test_eos_before_the_slice_still_resets(oracle):
    """An EOS just before the slice resets the first position in both forms."""
    case = next(c for c in SLICE_CASES if c["name"] == "cp_slice_after_eos_and_segment")
    start, end = case["slice"]
    glob = _unit_rows(oracle, case, 1, start, end)
    alone = _unit_rows(oracle, case, 1, start, end, whole_tokens=False)
    assert glob[0, 0] == 0 and alone[0, 0] == 0


@pytest.mark.parametrize("seed", [0, 1])
def test_slices_tile_the_sequence(oracle, seed):
    """Slices that cover the row end to end concatenate to the full hash,
    and the empty slice is empty."""
    wl = workloads.tiny()
    tok = wl.tokens(seed)
    S = tok.shape[1]
    args = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, wl.multipliers(), wl.primes,
            wl.offsets)
    full = oracle.hash(tok, *args)
    cuts = [0, 1, 37, 64, 65, S - 2, S]
    parts = [oracle.hash_global_slice(tok, a, b, *args) for a, b in zip(cuts, cuts[1:])]
    assert np.array_equal(np.concatenate(parts, axis=1), full)
    assert oracle.hash_global_slice(tok, 5, 5, *args).shape == (tok.shape[0], 0, len(wl.primes))
    with pytest.raises(ValueError):
        oracle.hash_global_slice(tok, 5, S + 1, *args)
