"""Host-side checks of the C ABI, written against any loaded copy of the
library's entry points: the HIP build (tests/test_abi.py) or the CPU build of
the same host code under ASan and UBSan (tests/test_abi_sanitized.py).  No
case reaches a kernel: each either fails validation or is empty, and every
device pointer passed is a fake address that must never be dereferenced.
Plain ctypes, no torch, so the sanitized child process can import it."""
import ctypes

from gram_hashed_embedding_amd import abi

i64arr = ctypes.c_int64 * 64
FAKE = ctypes.c_void_p(0x1000)        # never dereferenced: every case fails first
ALIGNED = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10008)
BAD_SIZE = (1 << 64) - 1              # engram_scatter_add_workspace's rejection


def _arr(vals):
    a = i64arr()
    for i, v in enumerate(vals):
        a[i] = v
    return a


def _ws(lib, n, rows, dim, mode):
    size = lib.engram_scatter_add_workspace(n, rows, dim, mode)
    assert size != BAD_SIZE
    return size


def case_status_strings_and_version(lib):
    assert lib.engram_abi_version() == abi.ABI_VERSION == 3
    assert lib.engram_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4):
        assert lib.engram_status_string(code) not in (b"ok", b"unknown status")
    assert lib.engram_status_string(7) == b"unknown status"


def _hash(lib, tokens=None, seg=None, batch=1, seq=4, n=3, J=2, mult=(1, 2, 3),
          primes=(5, 7, 11, 13), offs=(0, 5, 12, 23), rows=36, out=None):
    return lib.engram_hash(tokens, seg, batch, seq, n, J, 0, _arr(mult), _arr(primes),
                           _arr(offs), rows, out, None)


HASH_REJECTS = [
    dict(n=1), dict(n=9), dict(J=0), dict(n=8, J=10),            # orders / heads
    dict(primes=(5, 0, 11, 13)), dict(primes=(5, -7, 11, 13)),    # primes
    dict(offs=(0, 5, 12, -1)), dict(offs=(0, 5, 12, 30)),         # offsets past the table
    dict(batch=-1), dict(seq=-2), dict(rows=-5),
    dict(batch=1 << 40, seq=1 << 40),                            # size overflow
    dict(tokens=None, out=FAKE), dict(tokens=FAKE, out=None),     # null buffers
]


def case_hash_rejects(lib):
    for kwargs in HASH_REJECTS:
        args = dict(tokens=FAKE, out=FAKE)
        args.update(kwargs)
        assert _hash(lib, **args) == abi.ENGRAM_EINVAL, kwargs


def case_hash_empty_is_ok_without_launch(lib):
    assert _hash(lib, tokens=None, out=None, batch=0, seq=5) == abi.ENGRAM_OK
    assert _hash(lib, tokens=None, out=None, batch=3, seq=0) == abi.ENGRAM_OK


def case_hash_accepts_boundary_offsets(lib):
    # offset + prime == table_rows is allowed; an empty batch stops before launching
    assert _hash(lib, tokens=None, out=None, batch=0, offs=(0, 5, 12, 23), rows=36) == \
        abi.ENGRAM_OK
    assert _hash(lib, tokens=None, out=None, batch=0, offs=(0, 5, 12, 23), rows=35) == \
        abi.ENGRAM_EINVAL


def case_gather_rejects(lib):
    g = lib.engram_gather
    assert g(ALIGNED, 4, ALIGNED, 10, 12, ALIGNED, None, None) == abi.ENGRAM_EINVAL  # dim % 8
    assert g(ALIGNED, 4, ALIGNED, 10, 0, ALIGNED, None, None) == abi.ENGRAM_EINVAL
    assert g(ALIGNED, -1, ALIGNED, 10, 8, ALIGNED, None, None) == abi.ENGRAM_EINVAL
    assert g(None, 4, ALIGNED, 10, 8, ALIGNED, None, None) == abi.ENGRAM_EINVAL
    assert g(ALIGNED, 4, MISALIGNED, 10, 8, ALIGNED, None, None) == abi.ENGRAM_EALIGN
    assert g(ALIGNED, 4, ALIGNED, 10, 8, MISALIGNED, None, None) == abi.ENGRAM_EALIGN
    assert g(ALIGNED, 1 << 62, ALIGNED, 10, 8, ALIGNED, None, None) == abi.ENGRAM_EINVAL
    assert g(None, 0, None, 10, 8, None, None, None) == abi.ENGRAM_OK


def case_scatter_workspace_query(lib):
    w = lib.engram_scatter_add_workspace
    assert w(1000, 5000, 64, abi.SCATTER_ATOMIC) == 0
    sorted_bytes = w(1000, 5000, 64, abi.SCATTER_SORTED)
    assert sorted_bytes == w(1000, 5000, 64, abi.SCATTER_ROWSPARSE)
    assert sorted_bytes >= 16 * 1000            # keys and indices, twice
    assert w(2000, 5000, 64, abi.SCATTER_SORTED) > sorted_bytes
    assert w(0, 5000, 64, abi.SCATTER_SORTED) != BAD_SIZE
    for bad in [(10, 50, 12, 0), (10, 50, 4096, 0), (-1, 50, 8, 0), (10, 50, 8, 3),
                (10, 1 << 33, 8, 0)]:
        assert w(*bad) == BAD_SIZE, bad
    assert w(10, 1 << 33, 8, abi.SCATTER_ATOMIC) == 0   # atomic path has no key limit


def case_scatter_rejects(lib):
    s = lib.engram_scatter_add
    ws = _ws(lib, 100, 50, 8, 0)
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 50, 5, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert s(ALIGNED, 100, ALIGNED, 12, ALIGNED, 50, 0, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 50, 0, ALIGNED, ws - 1, None, None) == \
        abi.ENGRAM_EWORKSPACE
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 50, 0, None, 0, None, None) == \
        abi.ENGRAM_EWORKSPACE
    assert s(ALIGNED, 100, MISALIGNED, 8, ALIGNED, 50, 0, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EALIGN
    assert s(None, 100, ALIGNED, 8, ALIGNED, 50, 1, None, 0, None, None) == abi.ENGRAM_EINVAL
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 1 << 33, 0, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert s(None, 0, None, 8, None, 50, 0, None, 0, None, None) == abi.ENGRAM_OK
    r = lib.engram_scatter_add_rowsparse
    ws = _ws(lib, 100, 50, 8, 2)
    assert r(ALIGNED, 100, ALIGNED, 8, 50, ALIGNED, ALIGNED, None, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert r(ALIGNED, 100, ALIGNED, 8, 50, None, ALIGNED, ALIGNED, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert r(ALIGNED, 100, ALIGNED, 8, 50, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 16, None, None) == \
        abi.ENGRAM_EWORKSPACE


# The largest n the sorted path takes at each walker width (its apply launch
# holds at most 2^32 - 1 threads: 16 ids a walker of head_dim / 4 lanes, as a
# power of two up to 64; below 40 values the 32-bit ids bind first).
SORTED_LAUNCH_LIMITS = [(8, 4294967294), (32, 4294967294), (64, 4294901504),
                        (128, 2147450752), (136, 1073725376), (256, 1073725376),
                        (2048, 1073725376)]


def case_sorted_launch_limits(lib):
    w = lib.engram_scatter_add_workspace
    for dim, most in SORTED_LAUNCH_LIMITS:
        assert w(most, 1000, dim, abi.SCATTER_ROWSPARSE) != BAD_SIZE, dim
        assert w(most + 1, 1000, dim, abi.SCATTER_ROWSPARSE) == BAD_SIZE, dim
        assert w(most + 1, 1000, dim, abi.SCATTER_SORTED) == BAD_SIZE, dim
    n, big = 1073725376 + 1, 1 << 62
    assert lib.engram_scatter_plan(ALIGNED, n, 1000, 256, ALIGNED, big, None, None) == \
        abi.ENGRAM_EINVAL
    assert lib.engram_scatter_apply(ALIGNED, n, 256, 1000, ALIGNED, None, None, None, ALIGNED,
                                    big, None, None) == abi.ENGRAM_EINVAL
    assert lib.engram_scatter_apply_signsgd(ALIGNED, n, 256, 1000, ALIGNED, 0.5, ALIGNED, big,
                                            None, None) == abi.ENGRAM_EINVAL
    assert lib.engram_scatter_add(ALIGNED, n, ALIGNED, 256, ALIGNED, 1000, abi.SCATTER_SORTED,
                                  ALIGNED, big, None, None) == abi.ENGRAM_EINVAL
    assert lib.engram_scatter_add_rowsparse(ALIGNED, n, ALIGNED, 256, 1000, ALIGNED, ALIGNED,
                                            ALIGNED, ALIGNED, big, None, None) == \
        abi.ENGRAM_EINVAL


def case_plan_apply_reject(lib):
    ws = _ws(lib, 100, 50, 8, 2)
    pl, ap = lib.engram_scatter_plan, lib.engram_scatter_apply
    assert pl(ALIGNED, 100, 50, 12, ALIGNED, ws, None, None) == abi.ENGRAM_EINVAL   # dim % 8
    assert pl(None, 100, 50, 8, ALIGNED, ws, None, None) == abi.ENGRAM_EINVAL
    assert pl(ALIGNED, 100, 50, 8, ALIGNED, ws - 1, None, None) == abi.ENGRAM_EWORKSPACE
    assert pl(ALIGNED, 100, 50, 8, MISALIGNED, ws, None, None) == abi.ENGRAM_EWORKSPACE
    assert pl(None, 0, 50, 8, None, 0, None, None) == abi.ENGRAM_OK
    # exactly one output form
    assert ap(ALIGNED, 100, 8, 50, None, None, None, None, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ws, None,
              None) == abi.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, None, ALIGNED, None, ALIGNED, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EINVAL
    assert ap(MISALIGNED, 100, 8, 50, ALIGNED, None, None, None, ALIGNED, ws, None, None) == \
        abi.ENGRAM_EALIGN
    assert ap(ALIGNED, 100, 8, 50, ALIGNED, None, None, None, ALIGNED, 16, None, None) == \
        abi.ENGRAM_EWORKSPACE
    assert ap(None, 0, 8, 50, ALIGNED, None, None, None, None, 0, None, None) == abi.ENGRAM_OK


def case_hash_slice_rejects(lib):
    hs = lib.engram_hash_slice

    def call(start, end, gseq=8, batch=1, tokens=FAKE, out=FAKE):
        return hs(tokens, None, batch, gseq, start, end, 3, 2, 0, _arr((1, 2, 3)),
                  _arr((5, 7, 11, 13)), _arr((0, 5, 12, 23)), 36, out, None)
    for start, end in [(-1, 4), (5, 4), (0, 9), (9, 9)]:
        assert call(start, end) == abi.ENGRAM_EINVAL, (start, end)
    assert call(3, 3, tokens=None, out=None) == abi.ENGRAM_OK   # empty slice: no launch
    assert call(0, 8, batch=0, tokens=None, out=None) == abi.ENGRAM_OK
    assert call(0, 4, tokens=None) == abi.ENGRAM_EINVAL


def case_signsgd_rejects(lib):
    sg = lib.engram_signsgd_rowsparse
    E = abi
    assert sg(ALIGNED, ALIGNED, ALIGNED, 10, 12, ALIGNED, 50, 0.1, None, None) == E.ENGRAM_EINVAL
    assert sg(ALIGNED, ALIGNED, ALIGNED, -1, 8, ALIGNED, 50, 0.1, None, None) == E.ENGRAM_EINVAL
    assert sg(None, ALIGNED, ALIGNED, 10, 8, ALIGNED, 50, 0.1, None, None) == E.ENGRAM_EINVAL
    assert sg(ALIGNED, MISALIGNED, ALIGNED, 10, 8, ALIGNED, 50, 0.1, None, None) == \
        E.ENGRAM_EALIGN
    assert sg(ALIGNED, ALIGNED, ALIGNED, 10, 8, MISALIGNED, 50, 0.1, None, None) == \
        E.ENGRAM_EALIGN
    assert sg(None, None, None, 0, 8, None, 50, 0.1, None, None) == E.ENGRAM_OK
    assert sg(ALIGNED, ALIGNED, ALIGNED, 10, 8, ALIGNED, 1 << 60, 0.1, None, None) == \
        E.ENGRAM_EINVAL                                   # table size overflows
    ap = lib.engram_scatter_apply_signsgd
    ws = _ws(lib, 100, 50, 8, 2)
    assert ap(ALIGNED, 100, 12, 50, ALIGNED, 0.1, ALIGNED, ws, None, None) == E.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, None, 0.1, ALIGNED, ws, None, None) == E.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, MISALIGNED, 0.1, ALIGNED, ws, None, None) == E.ENGRAM_EALIGN
    assert ap(ALIGNED, 100, 8, 50, ALIGNED, 0.1, ALIGNED, 16, None, None) == E.ENGRAM_EWORKSPACE
    assert ap(None, 0, 8, 50, None, 0.1, None, 0, None, None) == E.ENGRAM_OK


def case_ple_conv_rejects(lib):
    cv = lib.engram_ple_conv

    def call(halo=None, halo_len=0, batch=2, seq=16, ch=16, K=4, d=3, x=ALIGNED, out=ALIGNED):
        return cv(x, halo, halo_len, None, ALIGNED, None, batch, seq, ch, K, d, out, None)
    assert call(ch=12) == abi.ENGRAM_EINVAL          # channels % 8
    assert call(ch=0) == abi.ENGRAM_EINVAL
    assert call(K=0) == abi.ENGRAM_EINVAL
    assert call(K=17) == abi.ENGRAM_EINVAL
    assert call(d=0) == abi.ENGRAM_EINVAL
    assert call(halo_len=9) == abi.ENGRAM_EINVAL     # a halo length without a halo
    assert call(halo_len=-1) == abi.ENGRAM_EINVAL
    assert call(x=None) == abi.ENGRAM_EINVAL
    assert call(x=MISALIGNED) == abi.ENGRAM_EALIGN
    assert call(halo=MISALIGNED, halo_len=9) == abi.ENGRAM_EALIGN
    assert call(seq=0, x=None, out=None) == abi.ENGRAM_OK
    assert call(seq=(1 << 62), halo=ALIGNED, halo_len=(1 << 62)) == abi.ENGRAM_EINVAL  # overflow
    assert call(ch=(1 << 61)) == abi.ENGRAM_EINVAL


def case_lookup_and_token_plan_reject(lib):
    lk = lib.engram_lookup

    def look(dim=8, table=ALIGNED, out=ALIGNED, rows=36, primes=(5, 7, 11, 13), tokens=FAKE):
        return lk(tokens, None, 1, 4, 3, 2, 0, _arr((1, 2, 3)), _arr(primes),
                  _arr((0, 5, 12, 23)), table, rows, dim, out, None, None)
    assert look(dim=12) == abi.ENGRAM_EINVAL
    assert look(primes=(5, 0, 11, 13)) == abi.ENGRAM_EINVAL
    assert look(rows=35) == abi.ENGRAM_EINVAL           # the last head does not fit
    assert look(table=None) == abi.ENGRAM_EINVAL
    assert look(tokens=None) == abi.ENGRAM_EINVAL
    assert look(table=MISALIGNED) == abi.ENGRAM_EALIGN
    assert look(out=MISALIGNED) == abi.ENGRAM_EALIGN
    pt = lib.engram_scatter_plan_tokens
    ws = _ws(lib, 24, 36, 8, 2)

    def plan(dim=8, wsb=ws, tokens=FAKE, work=ALIGNED, err=None):
        return pt(tokens, None, 1, 4, 3, 2, 0, _arr((1, 2, 3)), _arr((5, 7, 11, 13)),
                  _arr((0, 5, 12, 23)), 36, dim, work, wsb, err, None)
    assert plan(dim=12) == abi.ENGRAM_EINVAL
    assert plan(wsb=ws - 1) == abi.ENGRAM_EWORKSPACE
    assert plan(work=MISALIGNED) == abi.ENGRAM_EWORKSPACE
    assert plan(tokens=None) == abi.ENGRAM_EINVAL
    assert plan(dim=12, err=FAKE) == abi.ENGRAM_EINVAL


def case_lookup_slice_rejects(lib):
    ls = lib.engram_lookup_slice

    def look(start=1, end=3, gseq=4, dim=8, table=ALIGNED, out=ALIGNED, tokens=FAKE, batch=1):
        return ls(tokens, None, batch, gseq, start, end, 3, 2, 0, _arr((1, 2, 3)),
                  _arr((5, 7, 11, 13)), _arr((0, 5, 12, 23)), table, 36, dim, out, None, None)
    assert look(start=-1) == abi.ENGRAM_EINVAL
    assert look(start=3, end=2) == abi.ENGRAM_EINVAL       # slice reversed
    assert look(end=5) == abi.ENGRAM_EINVAL                # past the sequence
    assert look(dim=12) == abi.ENGRAM_EINVAL
    assert look(table=None) == abi.ENGRAM_EINVAL
    assert look(tokens=None) == abi.ENGRAM_EINVAL
    assert look(out=MISALIGNED) == abi.ENGRAM_EALIGN
    # empty slices and batches enqueue nothing
    assert look(start=2, end=2, table=None, out=None) == abi.ENGRAM_OK
    assert look(batch=0, tokens=None, table=None, out=None) == abi.ENGRAM_OK


def case_noalloc_limits(lib):
    """The allocation-free scatter-add takes any n whose workspace fits its
    fixed array (the e2e batch does) and rejects larger ones before any
    launch; its other checks are the row-sparse call's."""
    w = lib.engram_scatter_add_workspace
    assert w(1572864, 200000000, 256, abi.SCATTER_ROWSPARSE) <= abi.NOALLOC_SCRATCH_BYTES
    na = lib.engram_scatter_add_rowsparse_noalloc
    n = 4_000_000
    assert w(n, 200000000, 256, abi.SCATTER_ROWSPARSE) > abi.NOALLOC_SCRATCH_BYTES
    assert na(ALIGNED, n, ALIGNED, 256, 200000000, ALIGNED, ALIGNED, ALIGNED, None, None) == \
        abi.ENGRAM_EWORKSPACE
    assert na(ALIGNED, 100, ALIGNED, 12, 50, ALIGNED, ALIGNED, ALIGNED, None, None) == \
        abi.ENGRAM_EINVAL                                    # head_dim % 8
    assert na(ALIGNED, 100, ALIGNED, 8, 50, ALIGNED, ALIGNED, None, None, None) == \
        abi.ENGRAM_EINVAL                                    # no count
    assert na(None, 100, ALIGNED, 8, 50, ALIGNED, ALIGNED, ALIGNED, None, None) == \
        abi.ENGRAM_EINVAL
    assert na(ALIGNED, 100, MISALIGNED, 8, 50, ALIGNED, ALIGNED, ALIGNED, None, None) == \
        abi.ENGRAM_EALIGN


def _op(**fields):
    o = abi.EngramOp()
    for k, v in fields.items():
        setattr(o, k, v)
    return o


def _hash_op(op, **fields):
    """A lookup or token-plan op with valid hash arguments (3 orders, 2 heads
    per order, a 36-row table) and fake buffers."""
    base = dict(op=op, d_tokens=FAKE.value, batch=1, seq=4, ngram_size=3, heads_per_ngram=2,
                h_multipliers=_arr((1, 2, 3)), h_primes=_arr((5, 7, 11, 13)),
                h_offsets=_arr((0, 5, 12, 23)), table_rows=36, head_dim=8,
                d_table=ALIGNED.value, d_out=ALIGNED.value, d_workspace=ALIGNED.value,
                workspace_bytes=0)
    base.update(fields)
    return _op(**base)


def case_run_ops_rejects(lib):
    failed = ctypes.c_int64(99)
    ref = ctypes.byref(failed)
    assert lib.engram_run_ops(None, 0, ref) == abi.ENGRAM_OK and failed.value == -1
    assert lib.engram_run_ops(None, 1, ref) == abi.ENGRAM_EINVAL and failed.value == -1
    ops = (abi.EngramOp * 1)()
    assert lib.engram_run_ops(ops, -1, ref) == abi.ENGRAM_EINVAL and failed.value == -1
    bad_first = [
        _op(op=0), _op(op=7), _op(op=-1),                      # unknown op codes
        _op(op=abi.OP_RECORD), _op(op=abi.OP_WAIT),            # no event
        _hash_op(abi.OP_LOOKUP, ngram_size=1),                 # engram_lookup's own checks
        _hash_op(abi.OP_LOOKUP, d_out=None),
        _hash_op(abi.OP_PLAN_TOKENS, heads_per_ngram=0),       # engram_scatter_plan_tokens's
        _hash_op(abi.OP_PLAN_TOKENS, workspace_bytes=16),      # workspace too small: EWORKSPACE
        _op(op=abi.OP_APPLY, n=8, head_dim=7, table_rows=36),  # engram_scatter_apply's
        _op(op=abi.OP_APPLY_SIGNSGD, n=8, head_dim=8, table_rows=36),  # no table
    ]
    for o in bad_first:
        one = (abi.EngramOp * 1)(o)
        failed.value = 99
        rc = lib.engram_run_ops(one, 1, ref)
        assert rc in (abi.ENGRAM_EINVAL, abi.ENGRAM_EWORKSPACE), (o.op, rc)
        assert failed.value == 0, o.op
    # empty calls succeed without launching; the first failure's index comes back
    ok_empty = [_hash_op(abi.OP_LOOKUP, batch=0), _hash_op(abi.OP_PLAN_TOKENS, batch=0),
                _op(op=abi.OP_APPLY, n=0, head_dim=8, table_rows=36, d_grad_table=ALIGNED.value)]
    lst = (abi.EngramOp * 5)(*ok_empty, _op(op=abi.OP_WAIT), _op(op=abi.OP_LOOKUP))
    failed.value = 99
    assert lib.engram_run_ops(lst, 5, ref) == abi.ENGRAM_EINVAL and failed.value == 3
    failed.value = 99
    assert lib.engram_run_ops(lst, 3, ref) == abi.ENGRAM_OK and failed.value == -1
    assert lib.engram_run_ops(lst, 3, None) == abi.ENGRAM_OK


CASES = [v for k, v in sorted(globals().items()) if k.startswith("case_")]
