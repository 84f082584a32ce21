"""CPU check of the matrix-core kernel's LDS layouts: every staged element is
loaded once and lands where the fragment reads look for it, nothing leaves
its stage, and fragment reads are spread over the 64 LDS banks.  The index
functions are the kernel's own (k4_layout.h), compiled for the host."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_k4_layouts(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    if hipcc is None:
        pytest.skip("hipcc not available")
    exe = tmp_path / "k4_layout_check"
    subprocess.check_call([hipcc, "-O1", "-std=c++17", os.path.join(HERE, "k4_layout_check.hip"),
                           "-o", str(exe)], stderr=subprocess.DEVNULL)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout
