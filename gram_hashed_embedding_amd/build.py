"""Build libengram.so (HIP, gfx950) in-tree with hipcc.

    python -m gram_hashed_embedding_amd.build

compiles every csrc/*.hip into gram_hashed_embedding_amd/libengram.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
LIBRARY = PKG / "libengram.so"
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
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


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def build(verbose: bool = False) -> Path:
    """Compile all HIP sources into LIBRARY (always rebuilds)."""
    tmp = LIBRARY.with_suffix(".so.tmp")
    cmd = [hipcc(), *FLAGS, f"-I{INCLUDE}", f"-I{CSRC}",
           *map(str, sources()), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
