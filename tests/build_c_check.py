"""Build tests/c_abi_check (a plain HIP program that calls libgsample's C ABI
and compares with the oracle's C functions; no Python or torch in its
process).  Needs spatial_transformer_grid_amd/libgsample.so and
oracle/liboracle.so built first; the binary finds both through its rpath."""

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.cpp")
OUT = os.path.join(HERE, "c_abi_check")


def build() -> str:
    hipcc = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    pkg = os.path.join(ROOT, "spatial_transformer_grid_amd")
    orc = os.path.join(ROOT, "oracle")
    tmp = OUT + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-O2", "-std=c++17", "-Wall", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"),
           SRC, "-o", tmp, "-L", pkg, "-lgsample", "-L", orc, "-loracle",
           "-Wl,-rpath,$ORIGIN/../spatial_transformer_grid_amd", "-Wl,-rpath,$ORIGIN/../oracle"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building c_abi_check failed:\n%s" % (res.stdout + res.stderr))
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build())
