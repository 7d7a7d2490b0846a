"""Host-side check of the division by invariant integers the kernels use to
decode their work items (exact_attention_84_amd/csrc/fa_fastdiv.hpp):
tests/fastdiv_check.cpp compares it with plain integer division for every
divisor up to 4096, divisors around each power of two up to 2^31, 2000 random
divisors, and numerators at 0..2047, around multiples of the divisor, at
2^31 - 1 and at random below 2^31."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "fastdiv_check.cpp")
INC = os.path.join(ROOT, "exact_attention_84_amd", "csrc")


def test_fastdiv_matches_integer_division(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "fastdiv")
    subprocess.run([cxx, "-std=c++17", "-O2", "-I", INC, SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout
    assert r.stdout.strip().splitlines()[-1].startswith("checked ")
