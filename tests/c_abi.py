"""Build and run the plain C consumer of the library (tests/c_abi_consumer.c).

Test infrastructure: gcc compiles the C99 source against include/norm_bwd.h
and links it to the built library and the HIP runtime. The binary goes to
tests/_bin/ with a run path relative to itself, so the tree can move.
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCE = os.path.join(HERE, "c_abi_consumer.c")
BINARY = os.path.join(HERE, "_bin", "c_abi_consumer")
LIB_DIR = os.path.join(ROOT, "rmsnorm_backward_amd", "_lib")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    """Compile the consumer (always). Needs the built library."""
    if not os.path.exists(os.path.join(LIB_DIR, "libnorm_bwd.so")):
        raise RuntimeError("build the library first (rmsnorm_backward_amd._build)")
    os.makedirs(os.path.dirname(BINARY), exist_ok=True)
    tmp = BINARY + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROCM, "include"), SOURCE, "-o", tmp,
           "-L", LIB_DIR, "-lnorm_bwd", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../rmsnorm_backward_amd/_lib",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on {SOURCE}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, BINARY)
    return BINARY


def is_current() -> bool:
    """The binary exists and is newer than its source and the header (it
    links the library dynamically, so a rebuilt library needs no relink)."""
    if not os.path.exists(BINARY):
        return False
    t = os.path.getmtime(BINARY)
    return t >= os.path.getmtime(SOURCE) and \
        t >= os.path.getmtime(os.path.join(ROOT, "include", "norm_bwd.h"))


def run(*args: str, timeout: float = 120) -> subprocess.CompletedProcess:
    """Run the built consumer as a child process."""
    return subprocess.run([BINARY, *args], capture_output=True, text=True, timeout=timeout)
