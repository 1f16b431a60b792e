"""The library's host side -- every extern "C" entry point with its argument
checks (csrc/engram_host.cpp) -- built for the CPU with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, with stand-in launchers
(tests/host_launch_stub.cpp), and driven through every case of
tests/abi_cases.py in a child process.  The child aborts on the first
sanitizer report, or if an entry point launches work it should have refused."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gram_hashed_embedding_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")

CHILD = r"""
import ctypes, sys
sys.path.insert(0, {root!r})
from gram_hashed_embedding_amd import abi
from tests import abi_cases
lib = abi.declare(ctypes.CDLL({lib!r}))
for case in abi_cases.CASES:
    case(lib)
print("sanitized-ok", len(abi_cases.CASES))
"""


def _runtime(name):
    path = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_host_checks_under_asan_and_ubsan(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime here")
    lib = tmp_path / "libengram_hostcheck.so"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-shared", "-fPIC",
           "-Wall", "-Wextra", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "engram_host.cpp"),
           os.path.join(ROOT, "tests", "host_launch_stub.cpp"), "-o", str(lib)]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT, lib=str(lib))],
                         capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and "sanitized-ok" in res.stdout, \
        (res.stdout[-2000:], res.stderr[-4000:])
