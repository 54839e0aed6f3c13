"""Builds the C programs that the tests run, on the host, before any GPU run.

tests/_bin/c_dispatch_run: tests/c_dispatch_run.c compiled as C99 against the
public header and linked with the built dispatch library and the HIP runtime.
Its rpath is relative to its own location, so the tree can move as a whole.
"""

import os
import shutil
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "_bin")
DISPATCH_RUN = os.path.join(BIN, "c_dispatch_run")
ROCM = "/opt/rocm"


def build(verbose: bool = False) -> str:
    gcc = shutil.which("gcc")
    if gcc is None:
        raise RuntimeError("gcc not found")
    os.makedirs(BIN, exist_ok=True)
    tmp = DISPATCH_RUN + ".tmp"
    cmd = [gcc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror",
           # HIP's own headers need the platform macro from compilers other than hipcc.
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_dispatch_run.c"), "-o", tmp,
           "-L", os.path.join(ROOT, "moe_token_dispatch_amd"), "-lmoe_dispatch",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../moe_token_dispatch_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, DISPATCH_RUN)
    return DISPATCH_RUN


if __name__ == "__main__":
    print(build(verbose=True))
