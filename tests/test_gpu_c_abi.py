"""The C ABI from a plain HIP program, with no Python and no torch in its
process: tests/c_abi_check (built by build() from tests/c_abi_check.cpp)
allocates with hipMalloc on the ROCm install's HIP runtime, calls
gs_affine_grid, gs_grid_sample_2d (linear and nearest) and
gs_affine_grid_sample_fused, gs_resize (2x bilinear) and gs_deform_conv
(fp32 with a workspace) on seeded inputs, and compares with the oracle's C
functions: AffineGrid and nearest bit for bit, linear and Resize within 1e-5
of max|X|, DeformConv within 2e-5 of the sum of the absolute terms, fused
equal to the unfused pair bit for bit."""

import os
import subprocess

import pytest

from parity import note, torch_mod

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi_check")


def test_c_program_matches_the_oracle():
    if not torch_mod().cuda.is_available():
        pytest.skip("no GPU visible")
    assert os.path.exists(EXE), "tests/c_abi_check is not built (python tests/build_c_check.py)"
    note("C-ABI program %s" % EXE)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0 and "c abi check ok" in res.stdout, res.stdout + res.stderr
