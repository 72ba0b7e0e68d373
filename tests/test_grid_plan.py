"""Host-side check of the forward's work decomposition (CPU only).

tests/cpp/fwd_grid_check.cpp includes the same planner and grid-mapping
functions the kernels use (exact_tiled_attention_fa_amd/csrc/fa_launch.h) and
checks, over 25,752 shapes and three CU counts, that every visible key tile of
every query block is covered exactly once, that partial-result indices stay
inside the planned workspace, that the causal per-block splits fit one round
of work-groups, and that the combine reads exactly the partials written.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "cpp", "fwd_grid_check.cpp")
CSRC = os.path.join(ROOT, "exact_tiled_attention_fa_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the ROCm headers")
def test_forward_grid_covers_every_tile_once(tmp_path):
    exe = str(tmp_path / "fwd_grid_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE, "-I", CSRC, SRC,
                    "-o", exe], check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout[-2000:]
    assert "0 failures" in res.stdout
