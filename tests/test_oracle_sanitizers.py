"""The oracle's pin batteries on an AddressSanitizer + UndefinedBehaviorSanitizer
build of oracle/*.c (host code only).

The sources are compiled with -fsanitize=address,undefined and
-fno-sanitize-recover=all, and a child pytest process (the ASan runtime
preloaded, as a library loaded into Python needs) runs the dense-lattice
brute force, the closed forms (non-finite and huge locations included), the
page examples, the point-wise and type batteries and the planted-mistake
batteries, whose mutants are built with the same flags.  Any out-of-bounds
access, use of uninitialised stack memory through an index, signed overflow
or invalid conversion aborts the child.
"""

import os
import subprocess
import sys

import pytest

from conftest import ROOT

BATTERIES = ["test_oracle_bruteforce.py", "test_oracle_closed_forms.py", "test_oracle_pages.py",
             "test_oracle_points.py", "test_oracle_types.py", "test_oracle_mutants.py",
             "test_oracle_resize.py", "test_oracle_deform.py"]
FLAGS = "-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer -g"


def runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_pin_batteries_under_sanitizers(oracle_mod, tmp_path):
    asan = runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    lib = oracle_mod.build(out=str(tmp_path / "liboracle_san.so"), extra_flags=FLAGS.split())
    env = dict(os.environ)
    env.update({
        "ORACLE_LIB": lib,
        "ORACLE_EXTRA_CFLAGS": FLAGS,
        "LD_PRELOAD": asan,
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
    })
    tests = [os.path.join(ROOT, "tests", t) for t in BATTERIES]
    workers = str(max(1, min(8, len(os.sched_getaffinity(0)))))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-n", workers,
                        "-m", "not gpu", "-k", "not parallel"] + tests,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1800)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
