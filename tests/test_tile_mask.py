"""The attention kernel's tile visibility bits (csrc/tile_mask.hpp), compiled for
the host with the undefined-behaviour sanitizer, against a per-key brute force
of the mask definition (Clover page, causal mask construction: a node sees the
context, its ancestors and itself), over every tile offset, range end, lane
group and many ancestor-word shapes.  The replay of the kernel's earlier
per-element test agrees with the brute force wherever a range can end (k_end
<= ctx + 128; past that it reads the second ancestor word modulo 64) and
shifts by no more than 63: its bit arithmetic was right."""
import shutil
import subprocess
from pathlib import Path

import pytest

HERE = Path(__file__).resolve().parent


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_visibility_bits_under_ubsan(tmp_path):
    exe = tmp_path / "tile_mask_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-fsanitize=undefined",
                    "-fno-sanitize-recover=all", str(HERE / "tile_mask_check.cpp"), "-o",
                    str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "runtime error" not in res.stderr, res.stderr
    assert "(0 with k_end <= ctx + 128)" in res.stdout, res.stdout
