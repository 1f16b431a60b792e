"""GPU parity of the backward scatter-add against the oracle.

Sorted (deterministic) dense and row-sparse results must equal the oracle
bit for bit: both sum each row in fp64 and round once, and fp64 sums of
bf16 values are exact here.  The fp32 atomic variant adds every term into
the fp32 table in no fixed order.  Each of its elements must be within
1e-5 relative / 1e-6 absolute of the oracle, or, where a row has so many
terms that fp32 rounding alone exceeds that, within the worst-case error of
fp32 summation in any order: (k + 2) * 2^-24 * (|G| + sum |g_i|) for a row
with k terms (k roundings of the running sum, plus the oracle's own two).
How many elements fall outside 1e-5 / 1e-6, and the worst of them, is
reported as a warning (AtomicToleranceReport) in every run.

The sorted path's bit-exactness rests on one premise: each row's terms
and partial sums span at most 53 binary places, so fp64 sums them exactly
in any order.  test_wide_dynamic_range leaves that premise: gradients over
120 binades, summed in the kernels' order and in the oracle's, are held to
1e-5 relative (positive terms) or to the fp64 order bound (mixed signs),
and the elements that stop being bit-exact are counted.
"""
import warnings

import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, host_f32, needs_gpu, release
from tests.test_oracle_lookup import bits_to_f64

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

RTOL, ATOL = 1e-5, 1e-6


class AtomicToleranceReport(UserWarning):
    """Elements of the fp32-atomic scatter-add outside 1e-5 / 1e-6."""


class ExactnessReport(UserWarning):
    """Elements of the sorted scatter-add that are not bit-exact."""


def run_dense(ids, grads_dev, base_dev, mode):
    table = base_dev.clone()
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    E.engram_scatter_add(dev(ids), grads_dev, table, mode=mode, err_count=err)
    torch.cuda.synchronize()
    return table, int(err.item())


def run_sparse(ids, grads_dev, rows):
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    uid, uval, count = E.engram_scatter_add_rowsparse(dev(ids), grads_dev, rows, err_count=err)
    u = int(count.item())
    return uid[:u].cpu().numpy(), host_f32(uval[:u]), int(err.item())


def check_atomic(ids, gbits, base_h, got, want, rows, dim):
    valid = (ids >= 0) & (ids < rows)
    uniq, inv, cnt = np.unique(ids[valid], return_inverse=True, return_counts=True)
    absg = np.zeros((uniq.size, dim), dtype=np.float64)
    np.add.at(absg, inv, np.abs(bits_to_f64(gbits[valid])))
    diff = np.abs(got[uniq].astype(np.float64) - want[uniq])
    tol = ATOL + RTOL * np.abs(want[uniq].astype(np.float64))
    bound = (cnt[:, None] + 2) * 2.0 ** -24 * (np.abs(base_h[uniq]) + absg) * 1.01
    assert (diff <= np.maximum(tol, bound)).all()
    touched = np.zeros(rows, dtype=bool)
    touched[uniq] = True
    assert np.array_equal(got[~touched], base_h[~touched])
    beyond = diff > tol
    stats = {"elements": int(diff.size), "beyond_1e-5_1e-6": int(beyond.sum()),
             "worst_excess": float((diff - tol).max()) if diff.size else 0.0,
             "worst_rel": float((diff / np.maximum(np.abs(want[uniq]), 1e-30)).max())
             if diff.size else 0.0,
             "max_terms_per_row": int(cnt.max()) if cnt.size else 0}
    warnings.warn(AtomicToleranceReport(
        f"fp32 atomics, {rows} rows x {dim}: {stats['beyond_1e-5_1e-6']} of {stats['elements']} "
        f"elements outside 1e-5/1e-6 (worst excess {stats['worst_excess']:.3g}, worst relative "
        f"error {stats['worst_rel']:.3g}, up to {stats['max_terms_per_row']} terms per row); all "
        f"within the fp32 any-order bound"))
    return stats


def check_all_modes(oracle, ids, dim, rows, seed, base_std=1.0):
    grads = workloads.make_grads(ids.size, dim, seed, "cuda")
    gbits = bits(grads)
    base = workloads.make_grad_table(rows, dim, seed + 1 if base_std else None, "cuda")
    base_h = host_f32(base)
    want, bad = oracle.scatter_add_dense(ids, gbits, base_h)

    got, err = run_dense(ids, grads, base, E.SCATTER_SORTED)
    assert err == bad
    assert np.array_equal(host_f32(got).view(np.uint32), want.view(np.uint32))

    got_a, err_a = run_dense(ids, grads, base, E.SCATTER_ATOMIC)
    assert err_a == bad
    check_atomic(ids, gbits, base_h, host_f32(got_a), want, rows, dim)

    uid, uval, err_s = run_sparse(ids, grads, rows)
    want_uid, want_val, bad_s = oracle.scatter_add_rowsparse(ids, gbits, dim, rows)
    assert err_s == bad_s == bad
    assert np.array_equal(uid, want_uid)
    assert np.array_equal(uval.view(np.uint32), want_val.view(np.uint32))

    check_signsgd(oracle, ids, grads, want_uid, want_val, dim, rows, seed)


def check_signsgd(oracle, ids, grads, want_uid, want_val, dim, rows, seed, lr=2.0 ** -6):
    """The SignSGD step on a bf16 N(0, 0.02) table, fused into the apply and
    standalone on the row-sparse output, against the oracle bit for bit."""
    table0 = workloads.make_table(rows, dim, seed + 5, "cuda")
    want_t, _ = oracle.signsgd_rowsparse(want_uid, want_val, bits(table0), lr)
    fused = table0.clone()
    ws = E.engram_scatter_plan(dev(ids), rows, dim)
    E.engram_scatter_apply_signsgd(grads, ws, fused, lr)
    torch.cuda.synchronize()
    assert np.array_equal(bits(fused), want_t)
    del fused
    two_step = table0.clone()
    uid_d, uval_d, cnt_d = E.engram_scatter_add_rowsparse(dev(ids), grads, rows)
    E.engram_signsgd_rowsparse(uid_d, uval_d, cnt_d, two_step, lr)
    torch.cuda.synchronize()
    assert np.array_equal(bits(two_step), want_t)


def test_tiny_workload(oracle):
    wl = workloads.tiny()
    rows_ids = oracle.hash(wl.tokens(0), 3, 2, 0, wl.multipliers(), wl.primes, wl.offsets)
    check_all_modes(oracle, rows_ids.reshape(-1), wl.dim, wl.table_rows, 11)


def test_backward_workload(oracle):
    """The backward workload at full size: 262,144 lookups of Zipf(1.2)
    tokens into a 16.8M x 64 fp32 gradient table."""
    wl = workloads.backward()
    tok = wl.tokens(0)
    ids = oracle.hash(tok, wl.ngram_size, wl.heads_per_ngram, wl.eos_id, wl.multipliers(),
                      wl.primes, wl.offsets).reshape(-1)
    counts = np.bincount(ids)
    assert counts.max() > 100          # hot rows collide heavily
    check_all_modes(oracle, ids, wl.dim, wl.table_rows, 21)
    release()


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 63, 64, 65, 4095, 4096, 4097, 20011])
def test_ragged_counts(oracle, n):
    rng = np.random.Generator(np.random.PCG64(n))
    ids = np.minimum(rng.zipf(1.3, size=n) - 1, 499).astype(np.int64)
    check_all_modes(oracle, ids, 32, 500, 100 + n)


@pytest.mark.parametrize("dim", [8, 16, 24, 40, 128, 256, 520, 1024, 2048])
def test_dims(oracle, dim):
    rng = np.random.Generator(np.random.PCG64(dim))
    ids = np.minimum(rng.zipf(1.2, size=3000) - 1, 799).astype(np.int64)
    check_all_modes(oracle, ids, dim, 800, 200 + dim)


@pytest.mark.parametrize("pattern", ["one_row", "two_rows", "runs_at_range_edges",
                                     "sorted_runs", "all_distinct", "max_key",
                                     "every_length_sorted", "every_length_shuffled",
                                     "chunk_edges", "chunk_crossing"])
def test_run_structure(oracle, pattern):
    """Runs longer than a walker range, runs ending exactly on range edges,
    a single hot row spanning thousands of ranges."""
    rng = np.random.Generator(np.random.PCG64(len(pattern)))
    rows = 1 << 20
    if pattern == "one_row":
        ids = np.full(100_003, 777, dtype=np.int64)
    elif pattern == "two_rows":
        ids = rng.choice([5, rows - 1], size=50_000).astype(np.int64)
    elif pattern == "runs_at_range_edges":
        lens = rng.choice([1, 31, 32, 33, 64, 65, 96], size=600)
        ids = np.repeat(rng.permutation(rows)[:600], lens).astype(np.int64)
        ids = rng.permutation(ids)
    elif pattern == "sorted_runs":
        lens = rng.choice([1, 31, 32, 33, 64, 65, 96, 200], size=600)
        ids = np.repeat(np.sort(rng.permutation(rows)[:600]), lens).astype(np.int64)
    elif pattern == "all_distinct":
        ids = rng.permutation(rows)[:70_000].astype(np.int64)
    elif pattern == "chunk_edges":
        # long runs of one chunk, just over one, and of many (a chunk of the
        # apply is 512 sorted positions), among short ones
        lens = np.concatenate([[511, 512, 513, 1023, 1024, 1025, 1536, 2049, 5000, 18, 17, 33],
                               rng.integers(1, 40, size=400)])
        ids = np.repeat(rng.permutation(rows)[:lens.size], lens).astype(np.int64)
        ids = rng.permutation(ids)
    elif pattern == "chunk_crossing":
        # hundreds of long runs, each crossing one or two chunk boundaries:
        # several for every block of the apply's second launch
        lens = rng.integers(513, 1100, size=700)
        ids = np.repeat(rng.permutation(rows)[:lens.size], lens).astype(np.int64)
        ids = rng.permutation(ids)
    elif pattern.startswith("every_length"):
        # run lengths 1..50 in every phase against the sorted-order ranges
        lens = np.tile(np.arange(1, 51), 7)
        ids = np.repeat(np.sort(rng.permutation(rows)[:lens.size]), lens).astype(np.int64)
        if pattern.endswith("shuffled"):
            ids = rng.permutation(ids)
    else:  # the largest and smallest valid keys only
        ids = rng.choice([0, rows - 1], size=9_999).astype(np.int64)
    check_all_modes(oracle, ids, 64, rows, 300)


def _wide_bits(rng, n, dim, signed, binades=60):
    """bf16 bit patterns whose exponents spread over 2^-binades .. 2^binades
    (120 binades by default), random 7-bit mantissas, random signs when
    `signed`."""
    exp = rng.integers(127 - binades, 127 + binades + 1, size=(n, dim)).astype(np.uint16)
    man = rng.integers(0, 128, size=(n, dim)).astype(np.uint16)
    sign = (rng.integers(0, 2, size=(n, dim)).astype(np.uint16) << 15) if signed else 0
    return (sign | (exp << 7) | man).astype(np.uint16)


@pytest.mark.parametrize("kind", ["positive", "mixed", "cancelling"])
def test_wide_dynamic_range(oracle, kind):
    """Gradients over 120 binades: fp64 no longer sums a row exactly, so the
    kernels' order (walkers, then walker sums in a fixed order) and the
    oracle's (ascending flat index) may round differently.  Positive terms:
    every element within 1e-5 relative of the oracle (two fp64 orders differ
    by far less than fp32's last place; one fp32 rounding each).  Mixed
    signs (cancellation): within the bound of two fp64 orders of k terms,
    2 k 2^-53 sum |g|, plus one fp32 rounding each.  Cancelling: 300 rows of
    about 400 terms each (every row a long run, which the kernels sum in
    interleaved 16-term pieces combined in a fixed order), terms within 2^+-8,
    and in every row one +2^40 and one -2^40 term at random places, which
    cancel exactly; partial sums that hold one of them lose the small terms'
    low bits, so the two orders disagree (same bound).  Dense and row-sparse
    outputs, the same bits twice in a row, and the count of elements that are
    not bit-exact reported."""
    rng = np.random.Generator(np.random.PCG64(71 + ["positive", "mixed", "cancelling"].index(kind)))
    rows, dim = 3000, 64
    signed = kind != "positive"
    ids = np.minimum(rng.zipf(1.3, size=120_000) - 1, rows - 1).astype(np.int64)
    gbits = _wide_bits(rng, ids.size, dim, signed)
    if kind == "cancelling":
        rows = 300
        ids = rng.integers(0, rows, size=120_000).astype(np.int64)
        gbits = _wide_bits(rng, ids.size, dim, True, binades=8)
        big = np.uint16((127 + 40) << 7)  # 2^40 in bf16
        ids = np.concatenate([ids, np.arange(rows), np.arange(rows)]).astype(np.int64)
        gbits = np.concatenate([gbits, np.full((rows, dim), big, np.uint16),
                                np.full((rows, dim), big | np.uint16(0x8000), np.uint16)])
        order = rng.permutation(ids.size)
        ids, gbits = ids[order], np.ascontiguousarray(gbits[order])
    grads = torch.from_numpy(gbits.view(np.int16)).to("cuda").view(torch.bfloat16)
    base_h = np.zeros((rows, dim), dtype=np.float32)
    want, bad = oracle.scatter_add_dense(ids, gbits, base_h)
    got_t, err = run_dense(ids, grads, dev(base_h), E.SCATTER_SORTED)
    again, _ = run_dense(ids, grads, dev(base_h), E.SCATTER_SORTED)
    assert err == bad == 0
    assert torch.equal(got_t.view(torch.int32), again.view(torch.int32))
    uid, uval, err_s = run_sparse(ids, grads, rows)
    uniq, inv, cnt = np.unique(ids, return_inverse=True, return_counts=True)
    assert err_s == 0 and np.array_equal(uid, uniq)
    got = host_f32(got_t)
    assert np.array_equal(uval.view(np.uint32), got[uniq].view(np.uint32))
    absg = np.zeros((uniq.size, dim))
    np.add.at(absg, inv, np.abs(bits_to_f64(gbits)))
    w, g = want[uniq].astype(np.float64), got[uniq].astype(np.float64)
    diff = np.abs(g - w)
    if signed:
        tol = 2 * cnt[:, None] * 2.0 ** -53 * absg + 2 * 2.0 ** -24 * np.maximum(np.abs(w), np.abs(g))
    else:
        tol = RTOL * np.abs(w)
    assert (diff <= tol).all()
    inexact = int((got[uniq].view(np.uint32) != want[uniq].view(np.uint32)).sum())
    warnings.warn(ExactnessReport(
        f"sorted scatter-add, wide-range gradients ({kind}): "
        f"{inexact} of {diff.size} elements differ from the oracle's order in the last place or "
        f"more; worst |difference| / tolerance {float((diff / tol).max()):.3g}"))
    release()


def test_padding_and_invalid_ids(oracle):
    rng = np.random.Generator(np.random.PCG64(5))
    rows = 1000
    ids = rng.integers(0, rows, size=9000).astype(np.int64)
    ids[::7] = -1
    ids[::101] = rows
    ids[::211] = -5
    ids[::401] = 1 << 40
    check_all_modes(oracle, ids, 16, rows, 400)


def test_only_padding(oracle):
    ids = np.full(300, -1, dtype=np.int64)
    check_all_modes(oracle, ids, 16, 50, 401)


def test_tiny_tables(oracle):
    for rows in (1, 2, 3):
        ids = np.random.Generator(np.random.PCG64(rows)).integers(0, rows, size=777)
        check_all_modes(oracle, ids.astype(np.int64), 8, rows, 500 + rows)


def test_sorted_is_deterministic():
    wl = workloads.backward()
    rng = np.random.Generator(np.random.PCG64(9))
    ids = np.minimum(rng.zipf(1.1, size=200_000) - 1, 50_000).astype(np.int64)
    grads = workloads.make_grads(ids.size, 64, 9, "cuda")
    base = workloads.make_grad_table(50_001, 64, 10, "cuda")
    a, _ = run_dense(ids, grads, base, E.SCATTER_SORTED)
    b, _ = run_dense(ids, grads, base, E.SCATTER_SORTED)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    u1 = run_sparse(ids, grads, 50_001)
    u2 = run_sparse(ids, grads, 50_001)
    assert np.array_equal(u1[0], u2[0]) and np.array_equal(u1[1], u2[1])
    del wl


def test_empty():
    grads = torch.zeros((0, 8), dtype=torch.bfloat16, device="cuda")
    table = torch.ones((4, 8), dtype=torch.float32, device="cuda")
    ids = torch.zeros(0, dtype=torch.int64, device="cuda")
    E.engram_scatter_add(ids, grads, table)
    assert torch.equal(table, torch.ones_like(table))
    count = torch.full((1,), 9, dtype=torch.int64, device="cuda")
    E.engram_scatter_add_rowsparse(ids, grads, 4, num_unique=count)
    assert int(count.item()) == 0


def test_workspace_too_small_is_rejected():
    ids = torch.zeros(100, dtype=torch.int64, device="cuda")
    grads = torch.zeros((100, 8), dtype=torch.bfloat16, device="cuda")
    table = torch.zeros((4, 8), dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(E.EngramError) as info:
        E.engram_scatter_add(ids, grads, table, workspace=ws)
    assert info.value.status == E.ENGRAM_EWORKSPACE


def test_plan_apply_matches_one_call_and_reuses_plan(oracle):
    """The two-step form gives the one-call results bit for bit, and one plan
    serves several gradient tensors of the same ids (dense and row-sparse)."""
    wl = workloads.backward()
    ids = oracle.hash(wl.tokens(1), wl.ngram_size, wl.heads_per_ngram, wl.eos_id,
                      wl.multipliers(), wl.primes, wl.offsets).reshape(-1)
    ids_dev = dev(ids)
    rows, dim = wl.table_rows, wl.dim
    plan = E.engram_scatter_plan(ids_dev, rows, dim)
    for seed in (31, 32):
        grads = workloads.make_grads(ids.size, dim, seed, "cuda")
        base = workloads.make_grad_table(rows, dim, seed + 100, "cuda")
        one = base.clone()
        E.engram_scatter_add(ids_dev, grads, one)
        two = E.engram_scatter_apply(grads, plan, rows, grad_table=base.clone())
        assert torch.equal(one.view(torch.int32), two.view(torch.int32))
        u1, v1, c1 = E.engram_scatter_add_rowsparse(ids_dev, grads, rows)
        u2, v2, c2 = E.engram_scatter_apply(grads, plan, rows)
        n = int(c1.item())
        assert n == int(c2.item())
        assert torch.equal(u1[:n], u2[:n])
        assert torch.equal(v1[:n].view(torch.int32), v2[:n].view(torch.int32))
        want_uid, want_val, _ = oracle.scatter_add_rowsparse(ids, bits(grads), dim, rows)
        assert np.array_equal(u2[:n].cpu().numpy(), want_uid)
        assert np.array_equal(host_f32(v2[:n]).view(np.uint32), want_val.view(np.uint32))
    release()


def test_plan_on_side_stream(oracle):
    """Plan on a second stream, apply on the main one after an event."""
    wl = workloads.tiny()
    ids = oracle.hash(wl.tokens(2), 3, 2, 0, wl.multipliers(), wl.primes, wl.offsets).reshape(-1)
    ids_dev = dev(ids)
    grads = workloads.make_grads(ids.size, wl.dim, 77, "cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan = E.engram_scatter_plan(ids_dev, wl.table_rows, wl.dim)
        done = torch.cuda.Event()
        done.record(side)
    torch.cuda.current_stream().wait_event(done)
    uid, uval, count = E.engram_scatter_apply(grads, plan, wl.table_rows)
    n = int(count.item())
    want_uid, want_val, _ = oracle.scatter_add_rowsparse(ids, bits(grads), wl.dim, wl.table_rows)
    assert np.array_equal(uid[:n].cpu().numpy(), want_uid)
    assert np.array_equal(host_f32(uval[:n]).view(np.uint32), want_val.view(np.uint32))


@pytest.mark.parametrize("dim", [8, 24, 256])
@pytest.mark.parametrize("lr", [1e-6, 2.0 ** -8, 0.3])
def test_signsgd_standalone(oracle, dim, lr):
    """Given row-sparse input: fewer rows than the capacity, padding and
    out-of-range ids (skipped and counted), zero gradients (sign 0)."""
    rows, cap, u = 3000, 700, 611
    rng = np.random.Generator(np.random.PCG64(dim))
    ids = rng.choice(rows, cap, replace=False).astype(np.int64)
    ids[[3, 50]] = -1
    ids[[7, 400, 610]] = [rows, rows + 5, -9]
    ids[650] = 5        # past U: never read
    g = rng.normal(0, 1, (cap, dim)).astype(np.float32)
    g[rng.random((cap, dim)) < 0.2] = 0.0
    table = workloads.make_table(rows, dim, dim + 1, "cuda")
    want, bad = oracle.signsgd_rowsparse(ids[:u], g[:u], bits(table), lr)
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    count = torch.tensor([u], dtype=torch.int64, device="cuda")
    E.engram_signsgd_rowsparse(dev(ids), dev(g), count, table, lr, err_count=err)
    torch.cuda.synchronize()
    assert bad == 3 and int(err.item()) == bad
    assert np.array_equal(bits(table), want)


def test_signsgd_rejects():
    t = torch.zeros((10, 12), dtype=torch.bfloat16, device="cuda")   # 12 is not a multiple of 8
    ids = torch.zeros(4, dtype=torch.int64, device="cuda")
    with pytest.raises(E.EngramError):
        E.engram_signsgd_rowsparse(ids, torch.zeros((4, 12), device="cuda"),
                                   torch.zeros(1, dtype=torch.int64, device="cuda"), t, 0.1)


def random_ids(rng, n, rows):
    """A seeded mix of the id patterns the backward meets: uniform rows,
    Zipf-like hot rows (long runs after sorting, some spanning several
    walker ranges), a few rows repeated hundreds of times, padding (-1) and
    ids outside the table."""
    kind = rng.integers(0, 4)
    if kind == 0:
        ids = rng.integers(0, rows, n)
    elif kind == 1:
        ranks = np.minimum(rng.zipf(1.2, n), rows) - 1
        ids = rng.permutation(rows)[ranks] if rows <= 1 << 22 else ranks
    elif kind == 2:
        hot = rng.integers(0, rows, int(rng.integers(1, 6)))
        ids = np.where(rng.random(n) < 0.6, hot[rng.integers(0, hot.size, n)],
                       rng.integers(0, rows, n))
    else:
        ids = np.sort(rng.integers(0, rows, n))  # already sorted: runs at every boundary
    ids = ids.astype(np.int64)
    ids[rng.random(n) < 0.02] = -1
    bad = rng.random(n) < 0.005
    ids[bad] = rows + rng.integers(0, 1000, int(bad.sum()))
    return ids


@pytest.mark.parametrize("seed", range(16))
def test_random_sweep(oracle, seed):
    """Seeded random shapes: every output mode bit for bit (atomic within its
    bound), widths from 8 to 1024; even seeds take small tables (rows from 1
    up, log-uniform: long runs), odd seeds large ones (up to a few million
    rows: mostly distinct ids)."""
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    dim = int(rng.choice([8, 16, 24, 40, 64, 128, 256, 520, 1024]))
    max_rows = max(1, (1 << 23) // dim)
    if seed % 2 == 0:
        rows = int(min(max_rows, np.exp(rng.uniform(0, np.log(max_rows)))) + 1)
    else:
        rows = int(max_rows * rng.uniform(0.5, 1.0))
    n = int(rng.integers(1, 40000 if dim <= 256 else 6000))
    ids = random_ids(rng, n, rows)
    check_all_modes(oracle, ids, dim, rows, 500 + seed)
    release()


@pytest.mark.parametrize("tiles,extra", [(63, 4093), (64, 1), (100, 17), (127, 3), (128, 9)])
def test_sort_tile_sizes(oracle, tiles, extra):
    """Sorts around the size where the plan switches from half-size tiles
    (2048 keys, for sorts of fewer than 128 full tiles whose look-back words
    fit the workspace) to full 4096-key tiles, each with a ragged last tile
    and a few hot rows: every output mode bit for bit."""
    rng = np.random.Generator(np.random.PCG64(tiles * 10 + extra))
    n = tiles * 4096 + extra
    rows = 3_000_017
    ids = rng.integers(0, rows, n).astype(np.int64)
    hot = rng.integers(0, rows, 4)
    pick = rng.random(n) < 0.2
    ids[pick] = hot[rng.integers(0, 4, int(pick.sum()))]
    ids[rng.random(n) < 0.01] = -1
    check_all_modes(oracle, ids, 8, rows, 700 + tiles)
    release()


@pytest.mark.parametrize("dim", [8, 256, 512, 2048])
def test_long_runs_every_width(oracle, dim):
    """Long runs inside one chunk and across many, at row widths of one to
    eight quads per lane, in every output form."""
    rng = np.random.Generator(np.random.PCG64(dim))
    rows = 70_000
    lens = np.concatenate([[3000, 1025, 600, 512, 100, 40, 18], rng.integers(1, 30, size=300)])
    ids = np.repeat(rng.permutation(rows)[:lens.size], lens).astype(np.int64)
    ids = rng.permutation(ids)
    check_all_modes(oracle, ids, dim, rows, 700 + dim)


def test_apply_again_on_one_plan_with_chunks(oracle):
    """A plan whose long runs cross several chunks, applied three times in a
    row (each apply rewrites the per-chunk partial sums and owners the last
    one left): every apply equals the oracle."""
    rng = np.random.Generator(np.random.PCG64(77))
    rows, dim = 50_000, 64
    lens = np.concatenate([[4000, 1500, 700], rng.integers(1, 50, size=500)])
    ids = rng.permutation(np.repeat(rng.permutation(rows)[:lens.size], lens).astype(np.int64))
    grads = workloads.make_grads(ids.size, dim, 78, "cuda")
    want_uid, want_val, _ = oracle.scatter_add_rowsparse(ids, bits(grads), dim, rows)
    ws = E.engram_scatter_plan(dev(ids), rows, dim)
    for _ in range(3):
        err = torch.zeros(1, dtype=torch.int64, device="cuda")
        uid, uval, cnt = E.engram_scatter_apply(grads, ws, rows, err_count=err)
        torch.cuda.synchronize()
        u = int(cnt.item())
        assert int(err.item()) == 0 and u == want_uid.size
        assert np.array_equal(uid[:u].cpu().numpy(), want_uid)
        assert np.array_equal(host_f32(uval[:u]).view(np.uint32), want_val.view(np.uint32))
    release()


# (n, table_rows, hot): a plan of at most 262,144 ids sorts one pass on the
# top bits, then each bucket (about 512 ids) on the 9 to 24 bits below; hot
# rows past the 4096-key LDS buffer take the bucket's global-memory passes.
@pytest.mark.parametrize("n, rows, hot", [(4097, 1 << 12 | 5, 0), (20000, 20_000_000, 0),
                                          (100_000, 16_778_782, 6000),
                                          (262_144, 3_000_000_000, 0),
                                          (262_144, 16_778_782, 300)])
def test_id_plan_buckets_keep_the_sort_order(n, rows, hot):
    """The plan of n ids sorted by buckets holds the order of the full
    radix sort: the same ids followed by enough padding (-1, skipped) to
    pass 262,144 ids, which the passes of the full sort plan, give the same
    row-sparse sums bit for bit, with gradients whose sums depend on the
    order of every row's terms (+-2^40 among small terms)."""
    rng = np.random.Generator(np.random.PCG64(n + hot))
    ids = np.minimum(rng.zipf(1.2, n), rows - 1).astype(np.int64)
    ids = (ids * 2654435761) % rows  # spread the Zipf ranks over the table
    if hot:
        ids[rng.choice(n, hot, replace=False)] = rows // 3
    dim = 8
    pad = 262_145 - n
    exp = rng.integers(127 - 6, 127 + 7, (n + pad, dim)).astype(np.uint16)
    gb = ((rng.integers(0, 2, (n + pad, dim)).astype(np.uint16) << 15) | (exp << 7)
          | rng.integers(0, 128, (n + pad, dim)).astype(np.uint16))
    big = rng.random((n + pad, dim)) < 0.02
    gb[big] = (np.uint16((127 + 40) << 7) | (rng.integers(0, 2, int(big.sum())).astype(np.uint16)
                                              << 15))
    grads = torch.from_numpy(gb.view(np.int16)).to("cuda").view(torch.bfloat16)
    uid_b, val_b, err_b = run_sparse(ids, grads[:n].contiguous(), rows)
    padded = np.concatenate([ids, np.full(pad, -1, np.int64)])
    uid_f, val_f, err_f = run_sparse(padded, grads, rows)
    assert err_b == 0 and err_f == 0
    assert np.array_equal(uid_b, np.unique(ids))
    assert np.array_equal(uid_b, uid_f)
    assert np.array_equal(val_b.view(np.uint32), val_f.view(np.uint32))
    release()
