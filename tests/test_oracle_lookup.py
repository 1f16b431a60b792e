"""CPU pins for the oracle's gather and scatter-add (no GPU involved).

Gather is pinned to numpy fancy indexing (a library routine); scatter-add
to numpy's unbuffered ``np.add.at`` in fp64, to closed forms (distinct rows,
one shared row, integer-valued gradients) and to conservation of column
totals.
"""
import numpy as np
import pytest


def bf16_bits(rng, shape, scale=1.0):
    """Random bf16 bit patterns (round-to-nearest-even of float32 draws)."""
    f = (rng.standard_normal(size=shape) * scale).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits_exact(x):
    """bf16 bits of values that are exactly representable in bf16."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32)
    assert ((u & 0xFFFF) == 0).all()
    return (u >> 16).astype(np.uint16)


# ----------------------------------------------------------------- gather ---
@pytest.mark.parametrize("dim", [8, 32, 256])
def test_gather_matches_fancy_indexing(oracle, dim):
    rng = np.random.Generator(np.random.PCG64(dim))
    table = bf16_bits(rng, (997, dim))
    ids = rng.integers(0, 997, size=3001)
    out, bad = oracle.gather(ids, table)
    assert bad == 0
    assert np.array_equal(out, table[ids])


def test_gather_padding_and_invalid_rows(oracle):
    rng = np.random.Generator(np.random.PCG64(3))
    table = bf16_bits(rng, (50, 16))
    ids = np.array([3, -1, 49, 50, -2, 7, 1 << 40, -1], dtype=np.int64)
    out, bad = oracle.gather(ids, table)
    assert bad == 3                       # 50, -2 and 2^40; -1 is padding
    for i, r in enumerate(ids):
        if 0 <= r < 50:
            assert np.array_equal(out[i], table[r])
        else:
            assert not out[i].any()


def test_gather_empty(oracle):
    table = np.zeros((4, 8), dtype=np.uint16)
    out, bad = oracle.gather(np.zeros(0, dtype=np.int64), table)
    assert out.shape == (0, 8) and bad == 0


# ------------------------------------------------------------ scatter-add ---
def _addat_reference(ids, grads_bits, rows, dim, base):
    """fp64 accumulation with np.add.at (processes indices in order), one
    rounding to fp32, one fp32 add to the base table."""
    acc = np.zeros((rows, dim), dtype=np.float64)
    valid = (ids >= 0) & (ids < rows)
    np.add.at(acc, ids[valid], bits_to_f64(grads_bits[valid]))
    touched = np.zeros(rows, dtype=bool)
    touched[ids[valid]] = True
    out = base.astype(np.float32).copy()
    out[touched] = out[touched] + acc[touched].astype(np.float32)
    return out, touched, acc


@pytest.mark.parametrize("rows,n,dim", [(64, 2000, 8), (1000, 5000, 32), (37, 300, 64)])
def test_dense_matches_add_at(oracle, rows, n, dim):
    rng = np.random.Generator(np.random.PCG64(rows + n))
    # skewed ids so that rows collide many times
    ids = np.minimum(rng.zipf(1.3, size=n) - 1, rows - 1).astype(np.int64)
    grads = bf16_bits(rng, (n, dim))
    base = rng.standard_normal(size=(rows, dim)).astype(np.float32)
    got, bad = oracle.scatter_add_dense(ids, grads, base)
    want, touched, _ = _addat_reference(ids, grads, rows, dim, base)
    assert bad == 0
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert np.array_equal(got[~touched], base[~touched])


def test_dense_distinct_rows_is_plain_add(oracle):
    rng = np.random.Generator(np.random.PCG64(11))
    rows, dim = 500, 16
    ids = rng.permutation(rows)[:300].astype(np.int64)
    grads = bf16_bits(rng, (300, dim))
    base = rng.standard_normal(size=(rows, dim)).astype(np.float32)
    got, _ = oracle.scatter_add_dense(ids, grads, base)
    want = base.copy()
    want[ids] = base[ids] + bits_to_f64(grads).astype(np.float32)
    assert np.array_equal(got, want)


def test_dense_integer_gradients_exact(oracle):
    """Integer-valued gradients sum exactly in any precision, so the result
    is fixed by integer arithmetic alone."""
    rng = np.random.Generator(np.random.PCG64(12))
    rows, n, dim = 20, 4000, 8
    ids = rng.integers(0, rows, size=n).astype(np.int64)
    ints = rng.integers(-100, 101, size=(n, dim))
    grads = f64_to_bf16_bits_exact(ints)
    got, _ = oracle.scatter_add_dense(ids, grads, np.zeros((rows, dim), np.float32))
    want = np.zeros((rows, dim), dtype=np.int64)
    for i in range(n):
        want[ids[i]] += ints[i]
    assert np.array_equal(got, want.astype(np.float32))


def test_dense_one_shared_row(oracle):
    """All contributions on one row: the row receives their single sum,
    every other row is untouched."""
    rng = np.random.Generator(np.random.PCG64(13))
    n, dim = 1141, 32
    ids = np.full(n, 5, dtype=np.int64)
    grads = bf16_bits(rng, (n, dim))
    base = np.ones((9, dim), dtype=np.float32)
    got, _ = oracle.scatter_add_dense(ids, grads, base)
    s = bits_to_f64(grads).sum(axis=0)     # exact: bf16 sums fit fp64 here
    assert np.array_equal(got[5], (np.float32(1) + s.astype(np.float32)))
    assert (np.delete(got, 5, axis=0) == 1).all()


def test_dense_skips_padding_and_counts_invalid(oracle):
    rng = np.random.Generator(np.random.PCG64(14))
    ids = np.array([0, -1, 3, 4, 99, -7, 3], dtype=np.int64)
    grads = bf16_bits(rng, (7, 8))
    base = np.zeros((4, 8), dtype=np.float32)
    got, bad = oracle.scatter_add_dense(ids, grads, base)
    assert bad == 3                       # 4, 99 and -7 (table has 4 rows)
    g = bits_to_f64(grads)
    assert np.array_equal(got[0], g[0].astype(np.float32))
    assert np.array_equal(got[3], (g[2] + g[6]).astype(np.float32))
    assert not got[1].any() and not got[2].any()


def test_rowsparse_matches_dense(oracle):
    rng = np.random.Generator(np.random.PCG64(15))
    rows, n, dim = 3000, 20000, 16
    ids = np.minimum(rng.zipf(1.2, size=n) - 1, rows - 1).astype(np.int64)
    ids[::97] = -1
    grads = bf16_bits(rng, (n, dim))
    uid, vals, bad = oracle.scatter_add_rowsparse(ids, grads, dim, rows)
    assert bad == 0
    valid = ids[ids >= 0]
    assert np.array_equal(uid, np.unique(valid))          # ascending, unique
    dense, _ = oracle.scatter_add_dense(ids, grads, np.zeros((rows, dim), np.float32))
    assert np.array_equal(vals, dense[uid])
    _, _, acc = _addat_reference(ids, grads, rows, dim, np.zeros((rows, dim)))
    # conservation: column totals of the row sums equal the total of all
    # gradients (fp64 on both sides, within fp32 rounding of each row)
    tot = bits_to_f64(grads[ids >= 0]).sum(axis=0)
    assert np.allclose(vals.astype(np.float64).sum(axis=0), tot, rtol=1e-6, atol=1e-3)
    assert np.array_equal(vals, acc[uid].astype(np.float32))


def test_rowsparse_empty(oracle):
    uid, vals, bad = oracle.scatter_add_rowsparse(np.zeros(0, np.int64),
                                                  np.zeros((0, 8), np.uint16), 8, 10)
    assert uid.size == 0 and vals.shape == (0, 8) and bad == 0
