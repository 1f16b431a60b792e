"""Build libengram.so (HIP, gfx950) in-tree with hipcc.

    python -m gram_hashed_embedding_amd.build

compiles every csrc/*.hip with hipcc and the host-only csrc/*.cpp (the
entry points and their argument checks, plain C++) with ROCm's clang++, one
process per source, in parallel, and links them into
gram_hashed_embedding_amd/libengram.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libengram.so"
# the HBM streaming-copy probe the benchmark reports beside the roofline
PROBE_SOURCE = PKG / "probe" / "hbm_copy.hip"
PROBE_LIBRARY = PKG / "probe" / "libengram_probe.so"
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 vector ops (v_pk_*_f32) are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # hardware float atomics for the atomic scatter-add
    "-munsafe-fp-atomics",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libengram.so)")


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip")) + sorted(CSRC.glob("*.cpp"))


def host_cxx() -> str:
    for cand in (os.environ.get("ENGRAM_CXX"), "/opt/rocm/llvm/bin/clang++", shutil.which("g++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("no C++ compiler found for the host sources")


def _jobs() -> int:
    try:
        return max(1, min(int(os.environ.get("MAX_JOBS", "0")) or os.cpu_count() or 1, 16))
    except ValueError:
        return 4


def build_probe(verbose: bool = False) -> Path:
    """Compile the HBM streaming-copy probe into PROBE_LIBRARY."""
    tmp = PROBE_LIBRARY.with_suffix(".so.tmp")
    cmd = [hipcc(), *FLAGS, "-shared", str(PROBE_SOURCE), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROBE_LIBRARY)
    return PROBE_LIBRARY


def build(verbose: bool = False) -> Path:
    """Compile all HIP sources into LIBRARY, and the probe (always rebuilds)."""
    build_probe(verbose)
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="engram_build_") as tmpdir:
        objs = []

        def compile_one(src: Path) -> Path:
            obj = Path(tmpdir) / (src.stem + ".o")
            if src.suffix == ".cpp":
                cmd = [host_cxx(), *HOST_FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", str(src),
                       "-o", str(obj)]
            else:
                cmd = [cc, *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}", "-c", str(src), "-o", str(obj)]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj

        with ThreadPoolExecutor(max_workers=_jobs()) as pool:
            objs = list(pool.map(compile_one, sources()))
        tmp = LIBRARY.with_suffix(".so.tmp")
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
