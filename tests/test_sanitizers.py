"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The planner (``csrc/plan.cpp``, pure C++) is built with g++ together with
  ``tests/sanitize/plan_driver.cpp``, which sweeps valid and invalid plans and
  checks every invariant the kernels rely on.
* The oracle (``oracle/norm_oracle.c``) is built with gcc and both
  sanitizers, and the oracle's pin tests run against that build in a
  subprocess with the ASan runtime preloaded (Python itself is not
  instrumented; leak checking is off for that reason).
* A copy of the oracle with an off-by-one loop bound planted in it must be
  stopped by the same setup, so the harness is shown to catch an overrun.

The sanitizers apply to host code only; no GPU code is built here.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rmsnorm_backward_amd", "csrc")
ORACLE_SRC = os.path.join(ROOT, "oracle", "norm_oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="needs gcc and g++")


def _asan_runtime() -> str:
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("the gcc ASan runtime is not installed")
    return path


def _env(lib: str) -> dict:
    env = dict(os.environ)
    env.update(LD_PRELOAD=_asan_runtime(), NORM_ORACLE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return env


def _oracle_lib(src: str, out: str) -> str:
    subprocess.run(["gcc", *SAN, "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-shared",
                    "-fPIC", "-o", out, src, "-lm"], check=True)
    return out


def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_driver")
    subprocess.run(["g++", *SAN, "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
                    os.path.join(CSRC, "plan.cpp"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "abort_on_error=1",
                            "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    assert r.returncode == 0, r.stderr[-4000:]
    assert "plan driver:" in r.stdout and "runtime error" not in r.stderr


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = _oracle_lib(ORACLE_SRC, str(tmp_path / "liboracle_san.so"))
    env = _env(lib)
    # the instrumented copy is the one the tests load
    r = subprocess.run([sys.executable, "-c", "import oracle; print(oracle.default().path)"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == lib, r.stderr[-2000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_sanitizers_stop_a_planted_overrun(tmp_path):
    """The weight-gradient loop of a copy of the oracle reads one column past
    each row (j <= N): the instrumented build must abort on the first call."""
    src = open(ORACLE_SRC).read()
    old = ("        for (long j = 0; j < N; ++j) {\n"
           "            double xh = (x[r * N + j] - mu) * rs;\n"
           "            dgamma[j] += dy[r * N + j] * xh;")
    assert src.count(old) == 1
    bad = tmp_path / "norm_oracle_overrun.c"
    bad.write_text(src.replace(old, old.replace("j < N", "j <= N")))
    lib = _oracle_lib(str(bad), str(tmp_path / "liboracle_overrun.so"))
    code = ("import numpy as np, oracle\n"
            "x = np.ones((3, 200)); dy = np.ones((3, 200))\n"
            "oracle.bwd_wgrad('rmsnorm', x, dy, None, np.ones(3))\n"
            "print('not caught')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr, r.stderr[-2000:]
