"""GPU parity of the fused forward (engram_lookup: hash and gather in one
kernel) and of the plan made from the tokens (engram_scatter_plan_tokens)
against the oracle and against the separate calls: bit-exact."""
import numpy as np
import pytest
import torch

from gram_hashed_embedding_amd import workloads
from tests.gpu_helpers import bits, dev, host_f32, needs_gpu, release

pytestmark = needs_gpu
E = pytest.importorskip("gram_hashed_embedding_amd.engram")

# Every token plan and every apply of this file reports into an error
# counter, and each test ends by checking that none was bumped (no wait of a
# plan expired, and every apply found a complete plan of its sizes).
_COUNTERS = []


def plan_tokens(*args, **kwargs):
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    _COUNTERS.append(err)
    return E.engram_scatter_plan_tokens(*args, err_count=err, **kwargs)


def apply(*args, **kwargs):
    err = torch.zeros(1, dtype=torch.int64, device="cuda")
    _COUNTERS.append(err)
    return E.engram_scatter_apply(*args, err_count=err, **kwargs)


@pytest.fixture(autouse=True)
def no_plan_errors():
    _COUNTERS.clear()
    yield
    torch.cuda.synchronize()
    bumped = [int(c.item()) for c in _COUNTERS if int(c.item()) != 0]
    _COUNTERS.clear()
    assert not bumped, f"error counters bumped: {bumped}"


def hash_args(wl, mult):
    return (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, mult, wl.primes, wl.offsets)


def test_lookup_tiny_against_oracle(oracle):
    wl = workloads.tiny()
    table = workloads.make_table(wl.table_rows, wl.dim, wl.seed, "cuda")
    mult = wl.multipliers()
    for variant, segments in [(0, False), (1, True), (2, False)]:
        tok = wl.tokens(variant)
        seg = workloads.random_segments(tok.shape, 20, variant) if segments else None
        ids = torch.empty((tok.shape[0], tok.shape[1], len(wl.primes)), dtype=torch.int64,
                          device="cuda")
        out = E.engram_lookup(dev(tok), table, *hash_args(wl, mult),
                              seq_ids=None if seg is None else dev(seg), row_ids=ids)
        torch.cuda.synchronize()
        want_ids = oracle.hash(tok, *hash_args(wl, mult), seg)
        assert np.array_equal(ids.cpu().numpy(), want_ids)
        want, bad = oracle.gather(want_ids, bits(table))
        assert bad == 0
        assert np.array_equal(bits(out).reshape(-1, wl.dim), want)


@pytest.mark.parametrize("n", range(2, 9))
@pytest.mark.parametrize("dim", [8, 24, 64, 128, 256])
def test_lookup_every_order_and_width(oracle, n, dim):
    """Every ngram size (the kernel is compiled per size) and row widths with
    1, 3 (not a power of two), 8, 16 and 32 chunks (256, 256, 128, 64 and 32
    rows per block, the last block ragged), against the separate calls."""
    J = 2
    H = (n - 1) * J
    primes = workloads.primes_above(3000, H)
    offs = workloads.cumulative_offsets(primes)
    rows = sum(primes) + 5
    mult = workloads.seeded_multipliers(n, 40 + n)
    rng = np.random.Generator(np.random.PCG64(n * 100 + dim))
    tok = rng.integers(0, 50, (3, 97)).astype(np.int64)
    tok[rng.random(tok.shape) < 0.05] = 7
    seg = workloads.random_segments(tok.shape, 15, n)
    table = workloads.make_table(rows, dim, n + dim, "cuda")
    args = (n, J, 7, mult, primes, offs)
    ids = torch.empty((3, 97, H), dtype=torch.int64, device="cuda")
    out = E.engram_lookup(dev(tok), table, *args, seq_ids=dev(seg), row_ids=ids)
    sep_ids = E.engram_hash(dev(tok), *args, rows, seq_ids=dev(seg))
    sep_out = E.engram_gather(sep_ids, table)
    torch.cuda.synchronize()
    assert torch.equal(ids, sep_ids)
    assert torch.equal(out, sep_out)
    assert np.array_equal(ids.cpu().numpy(), oracle.hash(tok, *args, seg))


@pytest.mark.parametrize("name", ["tiny", "backward", "e2e"])
@pytest.mark.parametrize("segments", [False, True])
def test_token_plan_matches_id_plan_and_oracle(oracle, name, segments):
    wl = workloads.get(name)
    tok = wl.tokens(4)
    seg = workloads.random_segments(tok.shape, 200, wl.seed) if segments else None
    mult = wl.multipliers()
    args = hash_args(wl, mult)
    sd = None if seg is None else dev(seg)
    R = tok.size * len(wl.primes)
    grads = workloads.make_grads(R, wl.dim, wl.seed + 9, "cuda")
    ws_t = plan_tokens(dev(tok), wl.table_rows, wl.dim, *args, seq_ids=sd)
    uid_t, val_t, cnt_t = apply(grads, ws_t, wl.table_rows)
    ids = E.engram_hash(dev(tok), *args, wl.table_rows, seq_ids=sd)
    ws_i = E.engram_scatter_plan(ids.view(-1), wl.table_rows, wl.dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, wl.table_rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item())
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    if name != "e2e":   # the e2e backward is checked against the oracle at full size elsewhere
        want_uid, want_val, bad = oracle.scatter_add_rowsparse(ids.cpu().numpy().reshape(-1),
                                                               bits(grads), wl.dim,
                                                               wl.table_rows)
        assert bad == 0 and u == want_uid.size
        assert np.array_equal(uid_t[:u].cpu().numpy(), want_uid)
        assert np.array_equal(host_f32(val_t[:u]).view(np.uint32), want_val.view(np.uint32))
    del grads, ws_t, ws_i
    release()


@pytest.mark.parametrize("n,J", [(2, 1), (3, 4), (4, 3), (5, 16), (6, 2), (7, 5), (8, 9)])
def test_token_plan_every_order(n, J):
    """The plan made from the tokens equals the plan of engram_hash's ids for
    every ngram size, up to the most heads (64 = 4 orders x 16), with ragged
    tiles (a batch that is no multiple of the sort tile)."""
    H = (n - 1) * J
    primes = workloads.primes_above(5000, H)
    offs = workloads.cumulative_offsets(primes)
    rows = sum(primes) + 3
    mult = workloads.seeded_multipliers(n, 70 + n)
    rng = np.random.Generator(np.random.PCG64(n * 1000 + J))
    tok = rng.integers(0, 40, (3, 211)).astype(np.int64)
    tok[rng.random(tok.shape) < 0.03] = 5
    seg = workloads.random_segments(tok.shape, 30, n + J)
    args = (n, J, 5, mult, primes, offs)
    R = tok.size * H
    dim = 16
    grads = workloads.make_grads(R, dim, n + J, "cuda")
    ws_t = plan_tokens(dev(tok), rows, dim, *args, seq_ids=dev(seg))
    uid_t, val_t, cnt_t = apply(grads, ws_t, rows)
    ids = E.engram_hash(dev(tok), *args, rows, seq_ids=dev(seg))
    ws_i = E.engram_scatter_plan(ids.view(-1), rows, dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item()) and u > 0
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    assert torch.equal(uid_t[:u], torch.unique(ids))


@pytest.mark.parametrize("tokens", [1, 100, 4095, 4096, 4097, 8191, 8192, 8193, 9000])
def test_token_plan_sizes_keep_the_sort_order(tokens):
    """Small per-head segments are sorted by one block per head in LDS, larger
    ones by the multi-block sort: around both switches the plan from the
    tokens holds exactly the order of the plan of engram_hash's ids (equal
    rows in ascending flat index).  The gradients make the sums depend on
    that order: small terms with +-2^40 entries scattered among them, so a
    different order of any row's terms would change the result's bits."""
    n, J = 3, 4
    H = (n - 1) * J
    primes = workloads.primes_above(3000, H)
    offs = workloads.cumulative_offsets(primes)
    rows = sum(primes)
    mult = workloads.seeded_multipliers(n, 90)
    rng = np.random.Generator(np.random.PCG64(tokens))
    tok = np.minimum(rng.zipf(1.3, (1, tokens)), 60).astype(np.int64)   # hot rows
    args = (n, J, 0, mult, primes, offs)
    R, dim = tok.size * H, 16
    exp = rng.integers(127 - 6, 127 + 7, (R, dim)).astype(np.uint16)
    gb = ((rng.integers(0, 2, (R, dim)).astype(np.uint16) << 15) | (exp << 7)
          | rng.integers(0, 128, (R, dim)).astype(np.uint16))
    big = rng.random((R, dim)) < 0.02
    gb[big] = (np.uint16((127 + 40) << 7) | (rng.integers(0, 2, int(big.sum())).astype(np.uint16)
                                              << 15))
    grads = torch.from_numpy(gb.view(np.int16)).to("cuda").view(torch.bfloat16)
    ws_t = plan_tokens(dev(tok), rows, dim, *args)
    uid_t, val_t, cnt_t = apply(grads, ws_t, rows)
    ids = E.engram_hash(dev(tok), *args, rows)
    ws_i = E.engram_scatter_plan(ids.view(-1), rows, dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item()) and u > 0
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    release()


@pytest.mark.parametrize("case", ["zipf_21", "hot_21", "zipf_17", "hot_24", "zipf_25", "same_21",
                                  "short_21"])
def test_token_plan_buckets_keep_the_sort_order(case):
    """Per-head segments of more than 8192 keys on 17 to 24 bits are sorted by
    one pass on the top 8 bits and then bucket by bucket (in LDS, or through
    global memory for a bucket of more than 2048 keys: the "hot" cases hold a
    row of about 5,000 terms per head); 25 bits keep the passes of the full
    sort.  Either way the plan from the tokens holds exactly the order of the
    plan of engram_hash's ids, with gradients whose sums depend on the order
    of every row's terms (as in the test above).  "same": every token alike,
    so each head's keys are one row in one bucket; "short": 8193 tokens, one
    past the LDS plan's limit."""
    kind, b = case.split("_")
    n, J = 3, 2
    H = (n - 1) * J
    primes = workloads.primes_above(1 << (int(b) - 1), H)
    offs = workloads.cumulative_offsets(primes)
    rows = sum(primes)
    mult = workloads.seeded_multipliers(n, 91)
    rng = np.random.Generator(np.random.PCG64(int(b) * 7 + len(kind)))
    shape = (1, 8193) if kind == "short" else (2, 6100)
    tok = np.minimum(rng.zipf(1.2, shape), 5000).astype(np.int64)
    if kind == "hot":
        tok[rng.random(tok.shape) < 0.7] = 5
    if kind == "same":
        tok[:] = 7
    args = (n, J, 0, mult, primes, offs)
    R, dim = tok.size * H, 16
    exp = rng.integers(127 - 6, 127 + 7, (R, dim)).astype(np.uint16)
    gb = ((rng.integers(0, 2, (R, dim)).astype(np.uint16) << 15) | (exp << 7)
          | rng.integers(0, 128, (R, dim)).astype(np.uint16))
    big = rng.random((R, dim)) < 0.02
    gb[big] = (np.uint16((127 + 40) << 7) | (rng.integers(0, 2, int(big.sum())).astype(np.uint16)
                                              << 15))
    grads = torch.from_numpy(gb.view(np.int16)).to("cuda").view(torch.bfloat16)
    ws_t = plan_tokens(dev(tok), rows, dim, *args)
    uid_t, val_t, cnt_t = apply(grads, ws_t, rows)
    ids = E.engram_hash(dev(tok), *args, rows)
    ws_i = E.engram_scatter_plan(ids.view(-1), rows, dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item()) and u > 0
    if kind in ("hot", "same"):  # the hottest row outgrows the LDS buffer
        assert int(torch.unique(ids, return_counts=True)[1].max()) > 4096
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(uid_t[:u], torch.unique(ids))
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    release()


@pytest.mark.parametrize("seed", range(8))
def test_token_plan_buckets_random_sweep(seed):
    """A seeded sweep over the bucket plan's inputs: orders, heads per order,
    17 to 24 bits, 8193 to 16000 tokens a head, Zipf skew and a hot token's
    share; the plan from the tokens holds the order of the plan of the ids
    (sums that depend on the order of every row's terms)."""
    rng = np.random.Generator(np.random.PCG64(7000 + seed))
    n, J = int(rng.integers(2, 5)), int(rng.integers(1, 4))
    H = (n - 1) * J
    bits = int(rng.integers(17, 25))
    primes = workloads.primes_above((1 << (bits - 1)) + int(rng.integers(0, 1 << (bits - 2))), H)
    offs = workloads.cumulative_offsets(primes)
    rows = sum(primes)
    mult = workloads.seeded_multipliers(n, 100 + seed)
    batch = int(rng.integers(1, 3))
    seq = int(rng.integers(8193 // batch + 1, 16000 // batch))
    tok = np.minimum(rng.zipf(1.05 + rng.random(), (batch, seq)), 3000).astype(np.int64)
    tok[rng.random(tok.shape) < rng.random() * 0.5] = 11
    args = (n, J, 0, mult, primes, offs)
    R, dim = tok.size * H, 8
    exp = rng.integers(127 - 6, 127 + 7, (R, dim)).astype(np.uint16)
    gb = ((rng.integers(0, 2, (R, dim)).astype(np.uint16) << 15) | (exp << 7)
          | rng.integers(0, 128, (R, dim)).astype(np.uint16))
    big = rng.random((R, dim)) < 0.02
    gb[big] = (np.uint16((127 + 40) << 7) | (rng.integers(0, 2, int(big.sum())).astype(np.uint16)
                                              << 15))
    grads = torch.from_numpy(gb.view(np.int16)).to("cuda").view(torch.bfloat16)
    ws_t = plan_tokens(dev(tok), rows, dim, *args)
    uid_t, val_t, cnt_t = apply(grads, ws_t, rows)
    ids = E.engram_hash(dev(tok), *args, rows)
    ws_i = E.engram_scatter_plan(ids.view(-1), rows, dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item()) and u > 0
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    release()


@pytest.mark.parametrize("layout", ["ascending", "descending", "shuffled", "gap",
                                    "overlapping", "shared"])
def test_token_plan_head_layouts(layout):
    """The plan from the tokens sorts each head's rows on their own when the
    heads' row ranges are disjoint (in any order of offsets) and the whole key
    array otherwise; either way it equals the plan of engram_hash's ids.  Each
    head has several sort tiles, the last one ragged."""
    n, J = 3, 4
    H = (n - 1) * J
    primes = workloads.primes_above(60000, H)
    rng = np.random.Generator(np.random.PCG64(7 + len(layout)))
    order = list(range(H))
    if layout == "descending":
        order = order[::-1]
    elif layout == "shuffled":
        rng.shuffle(order)
    offs = [0] * H
    at = 0
    for h in order:   # back to back in the chosen order
        offs[h] = at
        at += primes[h]
    rows = at + 11
    if layout == "gap":   # a gap between two heads, the rest back to back
        offs = [o + (40 if h >= H // 2 else 0) for h, o in enumerate(offs)]
        rows += 40
    elif layout == "overlapping":   # head 1's range starts inside head 0's
        offs[1] = offs[0] + primes[0] // 2
    elif layout == "shared":   # two heads share one offset
        offs[3] = offs[2]
    mult = workloads.seeded_multipliers(n, 5)
    tok = rng.integers(0, 3000, (3, 5003)).astype(np.int64)
    tok[rng.random(tok.shape) < 0.01] = 9
    seg = workloads.random_segments(tok.shape, 400, 3)
    args = (n, J, 9, mult, primes, offs)
    R = tok.size * H
    dim = 8
    grads = workloads.make_grads(R, dim, 17, "cuda")
    ws_t = plan_tokens(dev(tok), rows, dim, *args, seq_ids=dev(seg))
    uid_t, val_t, cnt_t = apply(grads, ws_t, rows)
    ids = E.engram_hash(dev(tok), *args, rows, seq_ids=dev(seg))
    ws_i = E.engram_scatter_plan(ids.view(-1), rows, dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item()) and u > 0
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    assert torch.equal(uid_t[:u], torch.unique(ids))


@pytest.mark.parametrize("overlap", [False, True])
def test_plans_made_ahead_in_two_workspaces(overlap):
    """The schedule the bench times: the next batch's token plan made on a
    side stream into the other of two reused workspaces while this batch's
    lookup and apply run.  Every step's row-sparse output equals a fresh
    plan and apply of the same batch, bit for bit, so a reused workspace
    carries nothing over from the plan it held before.  Per-head segments,
    and (overlapping head ranges) one sort of all keys."""
    wl = workloads.backward()
    primes, offs = list(wl.primes), list(wl.offsets)
    if overlap:
        offs[1] = offs[0] + primes[0] // 3
    args = (wl.ngram_size, wl.heads_per_ngram, wl.eos_id, wl.multipliers(), primes, offs)
    rows, D = wl.table_rows, wl.dim
    toks = [dev(wl.tokens(k)) for k in range(3)]
    R = toks[0].numel() * len(primes)
    table = workloads.make_table(rows, D, 5, "cuda")
    grads = workloads.make_grads(R, D, 6, "cuda")
    out = torch.empty((R, D), dtype=torch.bfloat16, device="cuda")
    size = E.engram_scatter_add_workspace(R, rows, D, E.SCATTER_ROWSPARSE)
    wss = [torch.empty(size, dtype=torch.uint8, device="cuda") for _ in range(2)]
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    ev_plan = [torch.cuda.Event() for _ in range(2)]
    ev_apply = [torch.cuda.Event() for _ in range(2)]

    def plan(k):
        side.wait_event(ev_apply[k % 2])
        plan_tokens(toks[k % 3], rows, D, *args, workspace=wss[k % 2],
                                     stream=side)
        ev_plan[k % 2].record(side)

    got = []
    plan(0)
    for k in range(6):
        plan(k + 1)
        E.engram_lookup(toks[k % 3], table, *args, out=out)
        main.wait_event(ev_plan[k % 2])
        got.append(apply(grads, wss[k % 2], rows))
        ev_apply[k % 2].record(main)
    main.wait_stream(side)
    for k, (uid, val, cnt) in enumerate(got):
        ws = plan_tokens(toks[k % 3], rows, D, *args)
        uid_r, val_r, cnt_r = apply(grads, ws, rows)
        torch.cuda.synchronize()
        u = int(cnt_r.item())
        assert int(cnt.item()) == u and u > 0
        assert torch.equal(uid[:u], uid_r[:u])
        assert torch.equal(val[:u].view(torch.int32), val_r[:u].view(torch.int32))
    del got, grads, table, out
    release()


@pytest.mark.parametrize("seed", range(12))
def test_token_plan_random_sweep(seed):
    """Seeded random token plans against the plan of engram_hash's ids, bit
    for bit: ngram sizes 2..8, up to 64 heads, token counts from 1 to about
    40,000 (ragged tiles of either size), primes from tiny to 2^22, head
    offsets in a random order with random gaps, and on some seeds two
    heads' ranges overlapping (one sort of all keys)."""
    rng = np.random.Generator(np.random.PCG64(4200 + seed))
    n = int(rng.integers(2, 9))
    J = int(rng.integers(1, 64 // (n - 1) + 1))
    H = (n - 1) * J
    lo = int(np.exp(rng.uniform(np.log(3), np.log(1 << 22))))
    primes = workloads.primes_above(lo, H)
    order = rng.permutation(H)
    offs = [0] * H
    at = 0
    for h in order:
        at += int(rng.integers(0, 50))
        offs[h] = at
        at += primes[h]
    if seed % 3 == 2 and H > 1:
        a, b = int(order[0]), int(order[1])
        offs[b] = offs[a] + primes[a] // 2
    rows = at + int(rng.integers(1, 100))
    mult = workloads.seeded_multipliers(n, 300 + seed)
    batch = int(rng.integers(1, 4))
    seq = int(np.exp(rng.uniform(0, np.log(40000 // batch))))
    tok = rng.integers(0, int(rng.integers(2, 5000)), (batch, seq)).astype(np.int64)
    tok[rng.random(tok.shape) < 0.02] = 3
    seg = workloads.random_segments(tok.shape, int(rng.integers(5, 500)), seed) if seed % 2 else None
    sd = None if seg is None else dev(seg)
    args = (n, J, 3, mult, primes, offs)
    R = tok.size * H
    dim = 8
    grads = workloads.make_grads(R, dim, 50 + seed, "cuda")
    ws_t = plan_tokens(dev(tok), rows, dim, *args, seq_ids=sd)
    uid_t, val_t, cnt_t = apply(grads, ws_t, rows)
    ids = E.engram_hash(dev(tok), *args, rows, seq_ids=sd)
    ws_i = E.engram_scatter_plan(ids.view(-1), rows, dim)
    uid_i, val_i, cnt_i = apply(grads, ws_i, rows)
    torch.cuda.synchronize()
    u = int(cnt_t.item())
    assert u == int(cnt_i.item()) and u > 0
    assert torch.equal(uid_t[:u], uid_i[:u])
    assert torch.equal(val_t[:u].view(torch.int32), val_i[:u].view(torch.int32))
    assert torch.equal(uid_t[:u], torch.unique(ids))
    del grads, ws_t, ws_i
    release()
