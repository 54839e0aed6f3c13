"""Host code under the sanitizers, on the CPU.

- The dispatch library is rebuilt with UndefinedBehaviorSanitizer on its host
  code only (`-Xarch_host`; the device code is compiled as usual and never runs
  here), and the ABI tests, which drive every host-side argument check without
  touching a GPU, run against that build in a child process.
- The oracle is rebuilt with AddressSanitizer and UBSan, and its pins run
  against that build in a child process, so an out-of-bounds access or
  undefined behaviour in the reference the GPU is checked against fails here.

Any report aborts the child and fails the test.
"""

import glob
import os
import subprocess
import sys
import textwrap

import pytest

import oracle
from moe_token_dispatch_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ubsan_runtime():
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        return None
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        return None
    res = subprocess.run([clang, "--print-resource-dir"], capture_output=True, text=True)
    if res.returncode != 0:
        return None
    hits = glob.glob(os.path.join(res.stdout.strip(), "lib", "linux", "libclang_rt.ubsan_standalone-x86_64.so"))
    return hits[0] if hits else None


def test_abi_host_checks_clean_under_ubsan(tmp_path):
    runtime = _ubsan_runtime()
    if runtime is None:
        pytest.skip("no hipcc or no UBSan runtime next to it")
    lib = str(tmp_path / "libmoe_dispatch_ubsan.so")
    cmd = [B.hipcc(), *B.HIPCC_FLAGS, "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", B.INCLUDE, "-I", B.CSRC, "-o", lib, *[os.path.join(B.CSRC, s) for s in B.SOURCES]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    child = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import moe_token_dispatch_amd as M
        M.load_library({lib!r})
        import pytest
        sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                              {os.path.join(ROOT, "tests", "test_abi.py")!r}]))
    """)
    log = str(tmp_path / "ubsan")
    env = dict(os.environ, LD_PRELOAD=runtime, UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    run = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env, cwd=ROOT)
    reports = "".join(open(p).read() for p in glob.glob(log + "*"))
    assert run.returncode == 0 and not reports, (reports or run.stdout[-2000:] + run.stderr[-2000:])


def _gcc_runtime(name):
    res = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = res.stdout.strip()
    return path if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_pins_clean_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's ASan/UBSan runtimes are not installed")
    lib = str(tmp_path / "libdispatch_oracle_asan.so")
    res = subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC",
                          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                          "-I", os.path.dirname(oracle.LIB_PATH), "-o", lib,
                          os.path.join(os.path.dirname(oracle.LIB_PATH), "dispatch_oracle.c")],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_oracle_pins.py", "test_combine_check.py")]
    child = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import oracle
        oracle._lib = oracle.load_library({lib!r})
        import pytest
        sys.exit(pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider", *{tests!r}]))
    """)
    log = str(tmp_path / "asan")
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    run = subprocess.run([sys.executable, "-c", child], capture_output=True, text=True, env=env, cwd=ROOT)
    reports = "".join(open(p).read() for p in glob.glob(log + "*"))
    assert run.returncode == 0 and not reports, (reports or run.stdout[-2000:] + run.stderr[-2000:])
