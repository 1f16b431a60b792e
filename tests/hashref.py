"""Independent pure-Python formulation of the n-gram hash, for brute force.

Written from the same page statements as the C oracle but along a different
route, so that a slip in one is not repeated in the other:
  - the row is first cut into segments (a new segment starts at position 0,
    after every EOS, and wherever the packed segment id changes), and the
    window is read by position inside the segment (the oracle instead walks
    back one step at a time);
  - the mix is an exact Python integer, reduced to a signed 64-bit value at
    the end (the oracle wraps every product and partial sum in uint64);
  - the positive remainder is Python's floor-mod operator (the oracle
    corrects C's truncating remainder).
Only for small inputs: it is plain Python.
"""

FILL = 0


def to_int64(v: int) -> int:
    v %= 1 << 64
    return v - (1 << 64) if v >= 1 << 63 else v


def segment_starts(tokens, seg, eos):
    starts = []
    for j in range(len(tokens)):
        if (j == 0 or tokens[j - 1] == eos
                or (seg is not None and seg[j - 1] != seg[j])):
            starts.append(j)
    return starts


def windows(tokens, seg, eos, n):
    """window[t][k] = token k back from t inside t's segment, else FILL."""
    starts = segment_starts(tokens, seg, eos)
    out, si = [], 0
    for t in range(len(tokens)):
        while si + 1 < len(starts) and starts[si + 1] <= t:
            si += 1
        pos = t - starts[si]
        out.append([tokens[t - k] if k <= pos else FILL for k in range(n)])
    return out


def rows_for_sequence(tokens, seg, n, J, eos, mult, primes, offsets):
    result = []
    for w in windows(list(tokens), None if seg is None else list(seg), eos, n):
        row = []
        for g in range(2, n + 1):
            mix = to_int64(sum(int(w[k]) * int(mult[k]) for k in range(g)))
            for j in range(J):
                h = (g - 2) * J + j
                row.append(int(offsets[h]) + mix % int(primes[h]))
        result.append(row)
    return result
