"""CPU checks of the C ABI: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch.
No call here reaches a kernel (each either fails validation or is empty)."""
import ctypes

import pytest

e = pytest.importorskip("gram_hashed_embedding_amd.engram")

i64arr = ctypes.c_int64 * 64


def _arr(vals):
    a = i64arr()
    for i, v in enumerate(vals):
        a[i] = v
    return a


def test_every_declared_symbol_is_exported():
    names = e.declared_symbols()
    assert set(names) == {"engram_status_string", "engram_abi_version", "engram_hash",
                          "engram_gather", "engram_scatter_add_workspace",
                          "engram_scatter_add", "engram_scatter_add_rowsparse",
                          "engram_scatter_plan", "engram_scatter_apply",
                          "engram_hash_slice", "engram_signsgd_rowsparse",
                          "engram_scatter_apply_signsgd", "engram_ple_conv",
                          "engram_lookup", "engram_scatter_plan_tokens",
                          "engram_lookup_slice"}
    for name in names:
        assert hasattr(e._lib, name), name


def test_status_strings_and_version():
    assert e.engram_abi_version() == 1
    assert e.engram_status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert e.engram_status_string(code) not in ("ok", "unknown status")
    assert e.engram_status_string(7) == "unknown status"


def _hash(tokens=None, seg=None, batch=1, seq=4, n=3, J=2, mult=(1, 2, 3),
          primes=(5, 7, 11, 13), offs=(0, 5, 12, 23), rows=36, out=None):
    return e._lib.engram_hash(tokens, seg, batch, seq, n, J, 0, _arr(mult), _arr(primes),
                              _arr(offs), rows, out, None)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case fails first


@pytest.mark.parametrize("kwargs", [
    dict(n=1), dict(n=9), dict(J=0), dict(n=8, J=10),            # orders / heads
    dict(primes=(5, 0, 11, 13)), dict(primes=(5, -7, 11, 13)),    # primes
    dict(offs=(0, 5, 12, -1)), dict(offs=(0, 5, 12, 30)),         # offsets past the table
    dict(batch=-1), dict(seq=-2), dict(rows=-5),
    dict(batch=1 << 40, seq=1 << 40),                            # size overflow
    dict(tokens=None, out=FAKE), dict(tokens=FAKE, out=None),     # null buffers
])
def test_hash_rejects(kwargs):
    args = dict(tokens=FAKE, out=FAKE)
    args.update(kwargs)
    assert _hash(**args) == e.ENGRAM_EINVAL


def test_hash_empty_is_ok_without_launch():
    assert _hash(tokens=None, out=None, batch=0, seq=5) == e.ENGRAM_OK
    assert _hash(tokens=None, out=None, batch=3, seq=0) == e.ENGRAM_OK


def test_hash_accepts_boundary_offsets():
    # offset + prime == table_rows is allowed; an empty batch stops before launching
    assert _hash(tokens=None, out=None, batch=0, offs=(0, 5, 12, 23), rows=36) == e.ENGRAM_OK
    assert _hash(tokens=None, out=None, batch=0, offs=(0, 5, 12, 23), rows=35) == e.ENGRAM_EINVAL


ALIGNED = ctypes.c_void_p(0x10000)
MISALIGNED = ctypes.c_void_p(0x10008)


def test_gather_rejects():
    g = e._lib.engram_gather
    assert g(ALIGNED, 4, ALIGNED, 10, 12, ALIGNED, None, None) == e.ENGRAM_EINVAL  # dim % 8
    assert g(ALIGNED, 4, ALIGNED, 10, 0, ALIGNED, None, None) == e.ENGRAM_EINVAL
    assert g(ALIGNED, -1, ALIGNED, 10, 8, ALIGNED, None, None) == e.ENGRAM_EINVAL
    assert g(None, 4, ALIGNED, 10, 8, ALIGNED, None, None) == e.ENGRAM_EINVAL
    assert g(ALIGNED, 4, MISALIGNED, 10, 8, ALIGNED, None, None) == e.ENGRAM_EALIGN
    assert g(ALIGNED, 4, ALIGNED, 10, 8, MISALIGNED, None, None) == e.ENGRAM_EALIGN
    assert g(ALIGNED, 1 << 62, ALIGNED, 10, 8, ALIGNED, None, None) == e.ENGRAM_EINVAL
    assert g(None, 0, None, 10, 8, None, None, None) == e.ENGRAM_OK


def test_scatter_workspace_query():
    w = e.engram_scatter_add_workspace
    assert w(1000, 5000, 64, e.SCATTER_ATOMIC) == 0
    sorted_bytes = w(1000, 5000, 64, e.SCATTER_SORTED)
    assert sorted_bytes == w(1000, 5000, 64, e.SCATTER_ROWSPARSE)
    assert sorted_bytes >= 16 * 1000            # keys and indices, twice
    assert w(2000, 5000, 64, e.SCATTER_SORTED) > sorted_bytes
    assert w(0, 5000, 64, e.SCATTER_SORTED) >= 0
    for bad in [(10, 50, 12, 0), (10, 50, 4096, 0), (-1, 50, 8, 0), (10, 50, 8, 3),
                (10, 1 << 33, 8, 0)]:
        with pytest.raises(e.EngramError):
            w(*bad)
    assert w(10, 1 << 33, 8, e.SCATTER_ATOMIC) == 0   # atomic path has no key limit


def test_scatter_rejects():
    s = e._lib.engram_scatter_add
    ws = e.engram_scatter_add_workspace(100, 50, 8, 0)
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 50, 5, ALIGNED, ws, None, None) == e.ENGRAM_EINVAL
    assert s(ALIGNED, 100, ALIGNED, 12, ALIGNED, 50, 0, ALIGNED, ws, None, None) == e.ENGRAM_EINVAL
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 50, 0, ALIGNED, ws - 1, None, None) == \
        e.ENGRAM_EWORKSPACE
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 50, 0, None, 0, None, None) == e.ENGRAM_EWORKSPACE
    assert s(ALIGNED, 100, MISALIGNED, 8, ALIGNED, 50, 0, ALIGNED, ws, None, None) == \
        e.ENGRAM_EALIGN
    assert s(None, 100, ALIGNED, 8, ALIGNED, 50, 1, None, 0, None, None) == e.ENGRAM_EINVAL
    assert s(ALIGNED, 100, ALIGNED, 8, ALIGNED, 1 << 33, 0, ALIGNED, ws, None, None) == \
        e.ENGRAM_EINVAL
    assert s(None, 0, None, 8, None, 50, 0, None, 0, None, None) == e.ENGRAM_OK
    r = e._lib.engram_scatter_add_rowsparse
    ws = e.engram_scatter_add_workspace(100, 50, 8, 2)
    assert r(ALIGNED, 100, ALIGNED, 8, 50, ALIGNED, ALIGNED, None, ALIGNED, ws, None, None) == \
        e.ENGRAM_EINVAL
    assert r(ALIGNED, 100, ALIGNED, 8, 50, None, ALIGNED, ALIGNED, ALIGNED, ws, None, None) == \
        e.ENGRAM_EINVAL
    assert r(ALIGNED, 100, ALIGNED, 8, 50, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 16, None, None) == \
        e.ENGRAM_EWORKSPACE


def test_plan_apply_reject():
    ws = e.engram_scatter_add_workspace(100, 50, 8, 2)
    pl, ap = e._lib.engram_scatter_plan, e._lib.engram_scatter_apply
    assert pl(ALIGNED, 100, 50, 12, ALIGNED, ws, None, None) == e.ENGRAM_EINVAL   # dim % 8
    assert pl(None, 100, 50, 8, ALIGNED, ws, None, None) == e.ENGRAM_EINVAL
    assert pl(ALIGNED, 100, 50, 8, ALIGNED, ws - 1, None, None) == e.ENGRAM_EWORKSPACE
    assert pl(ALIGNED, 100, 50, 8, MISALIGNED, ws, None, None) == e.ENGRAM_EWORKSPACE
    assert pl(None, 0, 50, 8, None, 0, None, None) == e.ENGRAM_OK
    # exactly one output form
    assert ap(ALIGNED, 100, 8, 50, None, None, None, None, ALIGNED, ws, None) == e.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, ws, None) == \
        e.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, None, ALIGNED, None, ALIGNED, ALIGNED, ws, None) == \
        e.ENGRAM_EINVAL
    assert ap(MISALIGNED, 100, 8, 50, ALIGNED, None, None, None, ALIGNED, ws, None) == \
        e.ENGRAM_EALIGN
    assert ap(ALIGNED, 100, 8, 50, ALIGNED, None, None, None, ALIGNED, 16, None) == \
        e.ENGRAM_EWORKSPACE
    assert ap(None, 0, 8, 50, ALIGNED, None, None, None, None, 0, None) == e.ENGRAM_OK


def test_hash_slice_rejects():
    hs = e._lib.engram_hash_slice
    def call(start, end, gseq=8, batch=1, tokens=FAKE, out=FAKE):
        return hs(tokens, None, batch, gseq, start, end, 3, 2, 0, _arr((1, 2, 3)),
                  _arr((5, 7, 11, 13)), _arr((0, 5, 12, 23)), 36, out, None)
    for start, end in [(-1, 4), (5, 4), (0, 9), (9, 9)]:
        assert call(start, end) == e.ENGRAM_EINVAL, (start, end)
    assert call(3, 3, tokens=None, out=None) == e.ENGRAM_OK   # empty slice: no launch
    assert call(0, 8, batch=0, tokens=None, out=None) == e.ENGRAM_OK
    assert call(0, 4, tokens=None) == e.ENGRAM_EINVAL


def test_signsgd_rejects():
    sg = e._lib.engram_signsgd_rowsparse
    assert sg(ALIGNED, ALIGNED, ALIGNED, 10, 12, ALIGNED, 50, 0.1, None, None) == e.ENGRAM_EINVAL
    assert sg(ALIGNED, ALIGNED, ALIGNED, -1, 8, ALIGNED, 50, 0.1, None, None) == e.ENGRAM_EINVAL
    assert sg(None, ALIGNED, ALIGNED, 10, 8, ALIGNED, 50, 0.1, None, None) == e.ENGRAM_EINVAL
    assert sg(ALIGNED, MISALIGNED, ALIGNED, 10, 8, ALIGNED, 50, 0.1, None, None) == e.ENGRAM_EALIGN
    assert sg(ALIGNED, ALIGNED, ALIGNED, 10, 8, MISALIGNED, 50, 0.1, None, None) == e.ENGRAM_EALIGN
    assert sg(None, None, None, 0, 8, None, 50, 0.1, None, None) == e.ENGRAM_OK
    assert sg(ALIGNED, ALIGNED, ALIGNED, 10, 8, ALIGNED, 1 << 60, 0.1, None, None) == \
        e.ENGRAM_EINVAL                                   # table size overflows
    ap = e._lib.engram_scatter_apply_signsgd
    ws = e.engram_scatter_add_workspace(100, 50, 8, 2)
    assert ap(ALIGNED, 100, 12, 50, ALIGNED, 0.1, ALIGNED, ws, None) == e.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, None, 0.1, ALIGNED, ws, None) == e.ENGRAM_EINVAL
    assert ap(ALIGNED, 100, 8, 50, MISALIGNED, 0.1, ALIGNED, ws, None) == e.ENGRAM_EALIGN
    assert ap(ALIGNED, 100, 8, 50, ALIGNED, 0.1, ALIGNED, 16, None) == e.ENGRAM_EWORKSPACE
    assert ap(None, 0, 8, 50, None, 0.1, None, 0, None) == e.ENGRAM_OK


def test_ple_conv_rejects():
    cv = e._lib.engram_ple_conv
    def call(halo=None, halo_len=0, batch=2, seq=16, ch=16, K=4, d=3, x=ALIGNED, out=ALIGNED):
        return cv(x, halo, halo_len, None, ALIGNED, None, batch, seq, ch, K, d, out, None)
    assert call(ch=12) == e.ENGRAM_EINVAL          # channels % 8
    assert call(ch=0) == e.ENGRAM_EINVAL
    assert call(K=0) == e.ENGRAM_EINVAL
    assert call(K=17) == e.ENGRAM_EINVAL
    assert call(d=0) == e.ENGRAM_EINVAL
    assert call(halo_len=9) == e.ENGRAM_EINVAL     # a halo length without a halo
    assert call(halo_len=-1) == e.ENGRAM_EINVAL
    assert call(x=None) == e.ENGRAM_EINVAL
    assert call(x=MISALIGNED) == e.ENGRAM_EALIGN
    assert call(halo=MISALIGNED, halo_len=9) == e.ENGRAM_EALIGN
    assert call(seq=0, x=None, out=None) == e.ENGRAM_OK
    assert call(seq=(1 << 62), halo=ALIGNED, halo_len=(1 << 62)) == e.ENGRAM_EINVAL  # overflow
    assert call(ch=(1 << 61)) == e.ENGRAM_EINVAL


def test_lookup_and_token_plan_reject():
    lk = e._lib.engram_lookup
    def look(dim=8, table=ALIGNED, out=ALIGNED, rows=36, primes=(5, 7, 11, 13), tokens=FAKE):
        return lk(tokens, None, 1, 4, 3, 2, 0, _arr((1, 2, 3)), _arr(primes), _arr((0, 5, 12, 23)),
                  table, rows, dim, out, None, None)
    assert look(dim=12) == e.ENGRAM_EINVAL
    assert look(primes=(5, 0, 11, 13)) == e.ENGRAM_EINVAL
    assert look(rows=35) == e.ENGRAM_EINVAL           # the last head does not fit
    assert look(table=None) == e.ENGRAM_EINVAL
    assert look(tokens=None) == e.ENGRAM_EINVAL
    assert look(table=MISALIGNED) == e.ENGRAM_EALIGN
    assert look(out=MISALIGNED) == e.ENGRAM_EALIGN
    pt = e._lib.engram_scatter_plan_tokens
    ws = e.engram_scatter_add_workspace(24, 36, 8, 2)
    def plan(dim=8, wsb=ws, tokens=FAKE, work=ALIGNED):
        return pt(tokens, None, 1, 4, 3, 2, 0, _arr((1, 2, 3)), _arr((5, 7, 11, 13)),
                  _arr((0, 5, 12, 23)), 36, dim, work, wsb, None)
    assert plan(dim=12) == e.ENGRAM_EINVAL
    assert plan(wsb=ws - 1) == e.ENGRAM_EWORKSPACE
    assert plan(work=MISALIGNED) == e.ENGRAM_EWORKSPACE
    assert plan(tokens=None) == e.ENGRAM_EINVAL


def test_lookup_slice_rejects():
    ls = e._lib.engram_lookup_slice
    def look(start=1, end=3, gseq=4, dim=8, table=ALIGNED, out=ALIGNED, tokens=FAKE, batch=1):
        return ls(tokens, None, batch, gseq, start, end, 3, 2, 0, _arr((1, 2, 3)),
                  _arr((5, 7, 11, 13)), _arr((0, 5, 12, 23)), table, 36, dim, out, None, None)
    assert look(start=-1) == e.ENGRAM_EINVAL
    assert look(start=3, end=2) == e.ENGRAM_EINVAL       # slice reversed
    assert look(end=5) == e.ENGRAM_EINVAL                # past the sequence
    assert look(dim=12) == e.ENGRAM_EINVAL
    assert look(table=None) == e.ENGRAM_EINVAL
    assert look(tokens=None) == e.ENGRAM_EINVAL
    assert look(out=MISALIGNED) == e.ENGRAM_EALIGN
    # empty slices and batches enqueue nothing
    assert look(start=2, end=2, table=None, out=None) == e.ENGRAM_OK
    assert look(batch=0, tokens=None, table=None, out=None) == e.ENGRAM_OK


def test_host_constant_arrays():
    """The binding keeps one host array per set of hash constants: the same
    values (as a tuple, a list or a numpy array) give the same array, other
    values another one, and an array always holds exactly its values."""
    import numpy as np
    a = e._host_i64((5, -7, 2 ** 63 - 1), 3, "x")
    assert list(a) == [5, -7, 2 ** 63 - 1]
    assert e._host_i64([5, -7, 2 ** 63 - 1], 3, "x") is a
    assert e._host_i64(np.array([5, -7, 2 ** 63 - 1], dtype=np.int64), 3, "x") is a
    b = e._host_i64((5, -7, 3), 3, "x")
    assert b is not a and list(b) == [5, -7, 3] and list(a) == [5, -7, 2 ** 63 - 1]
    with pytest.raises(ValueError):
        e._host_i64((1, 2), 3, "x")
    for k in range(300):            # the cache stays bounded
        e._host_i64((k, k + 1), 2, "x")
    assert len(e._HOST_I64) <= 256
    assert list(e._host_i64((5, -7, 3), 3, "x")) == [5, -7, 3]
