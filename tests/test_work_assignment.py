"""GEMM work assignment with the tail split, checked on the host (CPU only).

Compiles tests/native/work_assignment_check.cpp against the library's GEMM
header with hipcc (host code only) and runs it: for the layer's GEMM shapes
and thousands of random tile counts, every (output tile, K step) is owned by
exactly one workgroup of the launch grid and every tail part writes the
partial slot the fixup kernel reads; and the float K-segment index of the
up-projection GEMM's concatenated operand is exact for every 64-aligned
offset below 2^24.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_work_assignment_covers_every_tile_step_once(tmp_path):
    if not (os.path.exists(HIPCC) or shutil.which(HIPCC)):
        pytest.skip("hipcc not available")
    exe = tmp_path / "wa"
    cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "grouped_expert_ffn_router_amd", "csrc"),
           os.path.join(ROOT, "tests", "native", "work_assignment_check.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    out = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout[-2000:]
