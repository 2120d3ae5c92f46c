"""Host check (no GPU) of the forward's query-head packing: compiles
tests/host/packed_heads_check.cpp against the header the kernel includes
(csrc/fwd_plan.hpp, fa::packed_head) with hipcc as a host program and runs
it. Every (b, h) of each KV group must be stored exactly once for group
sizes 1..8 and packs of 1, 2 and 4 heads."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


def test_packed_heads_exhaustive(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "packed_heads_check")
    src = os.path.join(ROOT, "tests", "host", "packed_heads_check.cpp")
    inc = os.path.join(ROOT, "block_sparse_masked_amd", "csrc")
    res = subprocess.run([hipcc, "-std=c++17", "-O1", "-I", inc, src, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
