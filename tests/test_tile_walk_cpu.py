"""The grouped GEMM's tile bookkeeping (csrc/tile_walk.h, the functions the
kernel's scheduler calls) compiled for the host and checked on the CPU: every
tile of consistent ragged offsets is visited exactly once, and offsets a caller
got wrong (negative, past n_max, decreasing, enormous) still give tiles whose
rows, gather rows and columns stay inside the buffers."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "mixture_experts_layer_16_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_tile_walk_bounds(tmp_path):
    exe = tmp_path / "tile_walk_check"
    src = os.path.join(HERE, "native", "tile_walk_check.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "0 failure(s)" in r.stdout
