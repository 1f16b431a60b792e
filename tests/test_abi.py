"""CPU checks of the C ABI of the built library: it loads, exports every
function the header declares, and rejects bad arguments on the host before
any launch.  The cases themselves are in tests/abi_cases.py (they also run
against a sanitized CPU build of the same host code)."""
import pytest

e = pytest.importorskip("gram_hashed_embedding_amd.engram")

from tests import abi_cases  # noqa: E402

EXPORTED = {"engram_status_string", "engram_abi_version", "engram_hash", "engram_gather",
            "engram_scatter_add_workspace", "engram_scatter_add", "engram_scatter_add_rowsparse",
            "engram_scatter_plan", "engram_scatter_apply", "engram_hash_slice",
            "engram_signsgd_rowsparse", "engram_scatter_apply_signsgd", "engram_ple_conv",
            "engram_lookup", "engram_scatter_plan_tokens", "engram_lookup_slice",
            "engram_scatter_add_rowsparse_noalloc", "engram_run_ops"}


def test_every_declared_symbol_is_exported():
    names = e.declared_symbols()
    assert set(names) == EXPORTED
    for name in names:
        assert hasattr(e._lib, name), name


@pytest.mark.parametrize("case", abi_cases.CASES, ids=lambda f: f.__name__[5:])
def test_abi_case(case):
    case(e._lib)


def test_launch_limits_of_the_gather_and_lookup():
    """Sizes whose kernel launch would pass 2^32 - 1 threads are refused by
    the library's launchers before any HIP call (the fake, aligned addresses
    are never read)."""
    lib, A = e._lib, abi_cases.ALIGNED
    most_blocks = (2 ** 32 - 1) // 256
    # gather, head_dim 8: 512 ids per 256-thread block; a table of no rows: 256
    assert lib.engram_gather(A, most_blocks * 512 + 1, A, 1000, 8, A, None, None) == \
        e.ENGRAM_EINVAL
    assert lib.engram_gather(A, most_blocks * 256 + 1, A, 0, 8, A, None, None) == \
        e.ENGRAM_EINVAL
    # fused lookup, head_dim 8: 256 lookups per block (one head: ngram 2, one head per order)
    one = abi_cases._arr((1, 3))
    seq = most_blocks * 256 + 1
    assert lib.engram_lookup(A, None, 1, seq, 2, 1, 0, one, abi_cases._arr((5,)),
                             abi_cases._arr((0,)), A, 5, 8, A, None, None) == e.ENGRAM_EINVAL


def test_binding_raises_on_bad_workspace_query():
    with pytest.raises(e.EngramError):
        e.engram_scatter_add_workspace(10, 50, 12, 0)


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



def test_op_struct_layout_matches_the_header(tmp_path):
    """The binding's engram_op (abi.EngramOp) has the header's size and
    field offsets, as a C compiler lays the struct out."""
    import ctypes
    import os
    import subprocess
    from gram_hashed_embedding_amd import abi
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    fields = [f for f, _ in abi.EngramOp._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"engram.h\"\n"
                   "int main(void) {\n  printf(\"%zu\\n\", sizeof(engram_op));\n"
                   + "".join(f'  printf("%zu\\n", offsetof(engram_op, {f}));\n' for f in fields)
                   + "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(root, "include"), str(src), "-o",
                    str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(abi.EngramOp)
    assert got[1:] == [getattr(abi.EngramOp, f).offset for f in fields]
