"""CPU checks of bench.py's host-side contract: more than one GPU is refused
with a message, and the algorithmic byte counts follow their definitions."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_e2e_step():
    sys.argv = ["bench.py"]
    import bench
    from gram_hashed_embedding_amd import workloads
    wl = workloads.e2e()
    N, R, D, U = wl.tokens_per_batch, wl.lookups, wl.dim, 1_362_632
    assert (N, R, D) == (65_536, 1_572_864, 256)
    fused = bench.algorithmic_bytes(wl, U)
    # forward: tokens in, table rows in, output out; the ids never reach memory
    assert fused["lookup"] == 8 * N + 2 * D * R + 2 * D * R
    # plan: it reads the tokens; apply: gradient rows in, fp32 sums and ids out
    assert fused["scatter_plan"] == 8 * N
    assert fused["scatter_apply"] == 2 * D * R + (4 * D + 8) * U
    assert sum(fused.values()) == 3_823_203_904
    sep = bench.algorithmic_bytes(wl, U, separate=True)
    assert sep["hash"] == 8 * N + 8 * R and sep["gather"] == 8 * R + 4 * D * R
    assert sep["scatter_plan"] == 8 * R


def test_code_digest_ignores_comments_only(tmp_path, monkeypatch):
    sys.argv = ["bench.py"]
    import bench
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("int f(int x) {  // twice\n  return 2 * x; /* doubled */\n}\n")
    b.write_text("/* header */ int f(int x) {\n\n  return 2 * x;   // another note\n}")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.code_digest(["a.hip"]) == bench.code_digest(["b.hip"])
    b.write_text("int f(int x) { return 3 * x; }")
    assert bench.code_digest(["a.hip"]) != bench.code_digest(["b.hip"])
