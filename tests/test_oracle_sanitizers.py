"""The oracle under UBSan and under ASan: int64 wraparound must be done
without undefined signed overflow (the page's hash relies on wrapping), and
no function may read or write outside its arrays.  Each sanitized build runs
in a child process, which aborts on the first report."""
import os
import subprocess
import sys

import pytest

from oracle import build
from oracle.engram_oracle import SOURCE

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
from oracle import Oracle
from tests import test_oracle_hash as H, test_oracle_lookup as L
o = Oracle({lib!r})
for s in range(6):
    H.test_wraparound_edge_values(o, s)
H.test_exhaustive_small_alphabet(o, 4, 2, 6, 7)
H.test_exhaustive_with_segments(o, 3, 2)
L.test_dense_matches_add_at(o, 64, 2000, 8)
L.test_rowsparse_matches_dense(o)
L.test_gather_padding_and_invalid_rows(o)
print("sanitized-ok")
"""


def _run_sanitized(tmp_path, flags, name, env=None):
    lib = build(SOURCE, tmp_path / name, extra_flags=flags)
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(lib))],
                         capture_output=True, text=True, timeout=600,
                         env=None if env is None else dict(os.environ, **env))
    assert res.returncode == 0 and "sanitized-ok" in res.stdout, res.stderr[-2000:]


def test_oracle_under_ubsan(tmp_path):
    _run_sanitized(tmp_path, ("-O1", "-fsanitize=undefined", "-fno-sanitize-recover=all"),
                   "liboracle_ubsan.so")


def test_oracle_under_asan(tmp_path):
    asan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not (os.path.isabs(asan) and os.path.exists(asan)):
        pytest.skip("gcc has no AddressSanitizer runtime here")
    _run_sanitized(tmp_path, ("-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address"),
                   "liboracle_asan.so",
                   env={"LD_PRELOAD": asan, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1"})
