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


SANITIZE = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs a host C++ compiler")
def test_tile_walk_bounds(tmp_path):
    # built with AddressSanitizer and UBSan where the host has them (any integer
    # overflow or out-of-bounds access in the bookkeeping aborts the check), else plain
    exe = tmp_path / "tile_walk_check"
    src = os.path.join(HERE, "native", "tile_walk_check.cpp")
    base = ["g++", "-std=c++17", "-I", CSRC, src, "-o", str(exe)]
    if subprocess.run(base + SANITIZE, capture_output=True).returncode != 0:
        subprocess.run(base + ["-O2"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "0 failure(s)" in r.stdout
    assert "runtime error" not in r.stderr, r.stderr[-2000:]
