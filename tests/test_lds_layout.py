"""Host check of the grouped LDS tile layout used by the head-dim-128 kernels.

Builds tests/lds_layout_check.cpp with the system C++ compiler against the
kernels' own index header (csrc/grp_layout.hpp) and runs it: copy placement,
operand addresses and bank-conflict freedom of both read patterns.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "flash_attention_transformers_amd", "csrc")


def test_grouped_layout_placement_reads_and_banks(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "lds_layout_check"
    subprocess.run([cxx, "-std=c++17", "-O1", "-I", CSRC, os.path.join(HERE, "lds_layout_check.cpp"),
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0 and out.stdout.strip() == "ok", out.stdout + out.stderr
