"""The OpenMP build of the oracle (the benchmark's all-core CPU baseline)
gives exactly what the serial build gives: the parallel loops only spread
independent tokens, lookups and distinct rows over threads."""
import numpy as np

from gram_hashed_embedding_amd import workloads
from oracle import default_oracle, openmp_oracle


def test_openmp_build_matches_serial():
    ser, par = default_oracle(), openmp_oracle()
    wl = workloads.backward()
    tok = wl.tokens(0)[:, :1500]
    seg = workloads.random_segments(tok.shape, 100, 3)
    args = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, wl.multipliers(), wl.primes,
            wl.offsets)
    ids = ser.hash(tok, *args, seg)
    assert np.array_equal(par.hash(tok, *args, seg), ids)
    rng = np.random.Generator(np.random.PCG64(5))
    rows, dim = 5000, 24
    flat = ids.reshape(-1) % rows
    flat[rng.random(flat.size) < 0.01] = -1
    flat[rng.random(flat.size) < 0.001] = rows + 3
    table = rng.integers(0, 1 << 16, (rows, dim), dtype=np.uint16)
    a, bad_a = ser.gather(flat, table)
    b, bad_b = par.gather(flat, table)
    assert np.array_equal(a, b) and bad_a == bad_b > 0
    grads = (rng.standard_normal((flat.size, dim)).astype(np.float32).view(np.uint32)
             >> 16).astype(np.uint16)
    base = rng.standard_normal((rows, dim)).astype(np.float32)
    da, bad_a = ser.scatter_add_dense(flat, grads, base.copy())
    db, bad_b = par.scatter_add_dense(flat, grads, base.copy())
    assert np.array_equal(da.view(np.uint32), db.view(np.uint32)) and bad_a == bad_b
    ua, va, _ = ser.scatter_add_rowsparse(flat, grads, dim, rows)
    ub, vb, _ = par.scatter_add_rowsparse(flat, grads, dim, rows)
    assert np.array_equal(ua, ub) and np.array_equal(va.view(np.uint32), vb.view(np.uint32))
    assert par.threads >= 1 and ser.threads == 1
