"""CPU pins for the oracle's hash (no GPU, no HIP code involved).

Each test ties the oracle to something other than itself: hand-written
windows from the pages' EOS and segment rules, an independent big-integer
formulation under exhaustive enumeration, closed forms, degenerate cases
and the constants printed on the API page.
"""
import itertools
import os

import numpy as np
import pytest

from gram_hashed_embedding_amd import workloads
from tests import hashref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "window_cases.txt")
INT64_MIN = -(1 << 63)
INT64_MAX = (1 << 63) - 1
P61 = (1 << 61) - 1          # Mersenne prime
P63 = (1 << 63) - 25         # largest prime below 2^63


def load_window_cases(path=GOLDEN):
    cases, cur = [], {}
    for raw in open(path):
        line = raw.strip()
        if line.startswith("#"):
            continue
        if not line:
            if cur:
                cases.append(cur)
                cur = {}
            continue
        key, _, val = line.partition(":")
        cur[key.strip()] = val.strip()
    if cur:
        cases.append(cur)
    out = []
    for c in cases:
        n = int(c["n"])
        toks = [int(x) for x in c["tokens"].split()]
        seg = None if c["seg"] == "-" else [int(x) for x in c["seg"].split()]
        exp = {k: [0 if x == "F" else int(x) for x in c[f"s{k}"].split()]
               for k in range(1, n)}
        sl = tuple(int(x) for x in c["slice"].split()) if "slice" in c else None
        out.append(dict(name=c["case"], n=n, eos=int(c["eos"]), tokens=toks,
                        seg=seg, expected=exp, slice=sl))
    return out


WINDOW_CASES = load_window_cases()


def test_golden_file_parses():
    assert len(WINDOW_CASES) >= 7
    for c in WINDOW_CASES:
        for k, v in c["expected"].items():
            assert len(v) == len(c["tokens"]), c["name"]


@pytest.mark.parametrize("case", WINDOW_CASES, ids=lambda c: c["name"])
def test_unit_multiplier_exposes_window(oracle, case):
    """With m = e_k (1 at index k, 0 elsewhere) and primes larger than every
    token, each head's row minus its offset is the token k back (or FILL)
    for orders above k, and 0 for orders that do not reach k."""
    n, J = case["n"], 2
    H = (n - 1) * J
    primes = [P61, 2147483647] * (n - 1)
    offsets = [1000 * (h + 1) for h in range(H)]
    tok = np.array([case["tokens"]], dtype=np.int64)
    seg = None if case["seg"] is None else np.array([case["seg"]], dtype=np.int64)
    for k in range(1, n):
        mult = np.zeros(n, dtype=np.int64)
        mult[k] = 1
        rows = oracle.hash(tok, n, J, case["eos"], mult, primes, offsets, seg)[0]
        for g in range(2, n + 1):
            for j in range(J):
                h = (g - 2) * J + j
                got = rows[:, h] - offsets[h]
                want = case["expected"][k] if g > k else [0] * len(case["tokens"])
                assert list(got) == want, (case["name"], k, g, j)


def test_current_token_multiplier(oracle):
    """m = e_0: every head sees the current token, whatever the history."""
    tok = np.array([[5, 9, 7, 9, 9, 3]], dtype=np.int64)
    rows = oracle.hash(tok, 3, 1, 9, [1, 0, 0], [P61, P61], [0, 50])[0]
    assert list(rows[:, 0]) == [5, 9, 7, 9, 9, 3]
    assert list(rows[:, 1] - 50) == [5, 9, 7, 9, 9, 3]


def _brute(oracle, tokens, seg, n, J, eos, mult, primes, offsets):
    got = oracle.hash(tokens, n, J, eos, mult, primes, offsets, seg)
    for b in range(tokens.shape[0]):
        want = hashref.rows_for_sequence(tokens[b], None if seg is None else seg[b],
                                         n, J, eos, mult, primes, offsets)
        assert got[b].tolist() == want, (tokens[b].tolist(),
                                         None if seg is None else seg[b].tolist())


SMALL_PRIMES = [3, 5, 7, 11, 13, 17, 19, 23, 29, 31, 37, 41]


@pytest.mark.parametrize("n,J,length,eos", [
    (2, 1, 6, 7), (2, 2, 6, 7), (3, 1, 6, 7), (3, 2, 6, 7),
    (4, 1, 6, 7), (4, 2, 6, 7), (3, 2, 8, 7), (3, 2, 6, 0),
])
def test_exhaustive_small_alphabet(oracle, n, J, length, eos):
    """Every sequence over {EOS, 1, 2, 3} of the given length, against the
    independent big-integer formulation."""
    alphabet = [eos, 1, 2, 3]
    tokens = np.array(list(itertools.product(alphabet, repeat=length)), dtype=np.int64)
    H = (n - 1) * J
    mult = workloads.seeded_multipliers(n, 31 + n * 10 + J)
    primes = SMALL_PRIMES[:H]
    offsets = workloads.cumulative_offsets(primes)
    _brute(oracle, tokens, None, n, J, eos, mult, primes, offsets)


@pytest.mark.parametrize("n,J", [(2, 2), (3, 2), (4, 1)])
def test_exhaustive_with_segments(oracle, n, J):
    """Every sequence over {EOS, 1, 2, 3} of length 5 crossed with every
    placement of packed-segment boundaries."""
    length, eos = 5, 7
    seqs = list(itertools.product([eos, 1, 2, 3], repeat=length))
    bounds = list(itertools.product([0, 1], repeat=length - 1))
    toks, segs = [], []
    for s in seqs:
        for bnd in bounds:
            toks.append(s)
            segs.append([0] + list(np.cumsum(bnd)))
    tokens = np.array(toks, dtype=np.int64)
    seg = np.array(segs, dtype=np.int64)
    H = (n - 1) * J
    mult = workloads.seeded_multipliers(n, 77 + n)
    primes = SMALL_PRIMES[-H:]
    offsets = workloads.cumulative_offsets(primes)
    _brute(oracle, tokens, seg, n, J, eos, mult, primes, offsets)


EDGE = [INT64_MIN, INT64_MIN + 1, -(1 << 62), -248044, -1, 0, 1, 2, 248044,
        (1 << 62), INT64_MAX - 1, INT64_MAX]


@pytest.mark.parametrize("seed", range(6))
def test_wraparound_edge_values(oracle, seed):
    """Tokens and multipliers at the edges of int64 (the mix wraps), primes
    from 2 up to the largest prime below 2^63, against big integers."""
    rng = np.random.Generator(np.random.PCG64(seed))
    n, J, eos = 4, 3, 248044
    H = (n - 1) * J
    tokens = np.array(rng.choice(EDGE, size=(16, 12)), dtype=np.int64)
    mult = np.array(rng.choice(EDGE + [23703573157769, -3], size=n), dtype=np.int64)
    primes = [2, 3, 1009, 20000003, P61, P63, 2147483647, 4294967311, 97][:H]
    offsets = [0] * H
    _brute(oracle, tokens, None, n, J, eos, mult, primes, offsets)
    seg = np.array(rng.integers(0, 2, size=(16, 12)).cumsum(axis=1), dtype=np.int64)
    _brute(oracle, tokens, seg, n, J, eos, mult, primes, offsets)


def test_page_multipliers_tiny(oracle):
    """The multipliers printed on the API page (section Data) on the tiny
    workload, against big integers.  With token ids below 248044 one
    product stays below 2^63 but their sum may wrap."""
    wl = workloads.tiny()
    tok = wl.tokens(0)
    mult = np.array(workloads.PAGE_LAYER_MULTIPLIERS, dtype=np.int64)
    _brute(oracle, tok, None, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult,
           wl.primes, wl.offsets)


def test_page_multipliers_wrap_for_real_ids():
    """Derived from the printed constants: a single product of a real token
    id with a multiplier stays in int64, a sum of three may not, so the
    page's 'signed int64 overflow' only bites under an additive mix."""
    m = workloads.PAGE_LAYER_MULTIPLIERS
    assert all(x % 2 == 1 for x in m)
    top = 248043
    assert max(m) * top < (1 << 63)
    assert sum(m) * top >= (1 << 63)


def test_zero_multipliers_give_offsets(oracle):
    wl = workloads.tiny()
    rows = oracle.hash(wl.tokens(0), 3, 2, 0, [0, 0, 0], wl.primes, wl.offsets)
    assert (rows == np.array(wl.offsets)).all()


def test_unit_primes_give_offsets(oracle):
    tok = np.arange(-50, 50, dtype=np.int64).reshape(2, 50)
    rows = oracle.hash(tok, 3, 2, 0, [INT64_MAX, -7, 123], [1, 1, 1, 1], [4, 9, 16, 25])
    assert (rows == np.array([4, 9, 16, 25])).all()


def test_rows_stay_in_head_range(oracle):
    """Every row lies in [offset, offset + prime) of its head."""
    for name in ("tiny", "medium", "backward"):
        wl = workloads.get(name)
        rows = oracle.hash(wl.tokens(0), wl.ngram_size, wl.heads_per_ngram, wl.eos_id,
                           wl.multipliers(), wl.primes, wl.offsets)
        off = np.array(wl.offsets)
        pr = np.array(wl.primes)
        assert (rows >= off).all() and (rows < off + pr).all(), name
        # every head is used and heads are not all equal (the hash spreads)
        assert len(np.unique(rows[..., 0])) > rows.shape[1] // 4


def test_heads_grouped_by_order(oracle):
    """Bigram heads come first, then trigram heads.  With m[2] = 0 the
    trigram mix equals the bigram mix, so with the same primes in both
    groups the two groups coincide; changing m[2] changes only the trigram
    group."""
    wl = workloads.medium()
    tok = wl.tokens(0)[:, :512]
    J = 3
    primes = [1048583, 1048589, 1048601] * 2
    offs = [0] * 6
    m = wl.multipliers()
    m0 = m.copy()
    m0[2] = 0
    rows0 = oracle.hash(tok, 3, J, wl.eos_id, m0, primes, offs)
    assert (rows0[..., :J] == rows0[..., J:]).all()
    rows1 = oracle.hash(tok, 3, J, wl.eos_id, m, primes, offs)
    assert (rows1[..., :J] == rows0[..., :J]).all()
    assert (rows1[..., J:] != rows0[..., J:]).mean() > 0.5


def test_rejects_bad_arguments(oracle):
    tok = np.zeros((1, 4), dtype=np.int64)
    with pytest.raises(ValueError):
        oracle.hash(tok, 1, 1, 0, [1], [], [])
    with pytest.raises(ValueError):
        oracle.hash(tok, 2, 1, 0, [1, 1], [0], [0])


def test_page_constants_reconstruct():
    """Derived facts from the printed constants (API page, section Data):
    the 8 printed moduli are the first 8 primes above 2*10^7; the printed
    offsets are their running sums; 16 such primes, packed and rounded up
    to a multiple of 128, give exactly the printed padded row count; at a
    row width of 160 bf16 that is the 102.4 GB table the page names."""
    printed = workloads.PAGE_HEAD_VOCAB_SIZES_PRINTED
    assert list(printed) == workloads.primes_above(20_000_000, 8)
    assert list(workloads.PAGE_HEAD_OFFSETS_PRINTED) == workloads.cumulative_offsets(printed)
    sixteen = workloads.primes_above(20_000_000, 16)
    offs = workloads.cumulative_offsets(sixteen)
    assert str(offs[8]).startswith("160") and offs[8] == 160000374
    total = sum(sixteen)
    assert total == 320001446
    assert ((total + 127) // 128) * 128 == workloads.PAGE_PADDED_ROWS
    assert workloads.PAGE_PADDED_ROWS * 160 * 2 == 102_400_491_520
