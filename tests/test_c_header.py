"""The public header from a C caller, on the CPU.

tests/c_abi_probe.c is compiled as C99 with -Wall -Wextra -Werror against
include/moe_dispatch.h and linked with the built library. What it prints (the
size and every field offset of each struct, and the host-only calls' results)
must equal what the Python binding's ctypes structures and calls give, so a C
caller and the binding see one ABI. No GPU is touched.
"""

import ctypes
import os
import shutil
import subprocess

import pytest

import moe_token_dispatch_amd as M
from moe_token_dispatch_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "moe_token_dispatch_amd")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def probe(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.isdir(ROCM_INCLUDE):
        pytest.skip("gcc or the ROCm headers are not installed")
    M.load_library()  # the library is built
    exe = str(tmp_path_factory.mktemp("cabi") / "c_abi_probe")
    # HIP's own headers need the platform macro from compilers other than hipcc.
    build = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                            "-I", ROCM_INCLUDE, "-I", os.path.join(ROOT, "include"),
                            os.path.join(ROOT, "tests", "c_abi_probe.c"), "-o", exe,
                            "-L", PKG, "-lmoe_dispatch", f"-Wl,-rpath,{PKG}"],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr
    out = {}
    for line in run.stdout.splitlines():
        key, _, val = line.partition(" ")
        out[key] = val
    return out


STRUCTS = {
    "dispatch_problem_t": B.Problem,
    "dispatch_layout_t": B.LayoutPtrs,
    "dispatch_expand_problem_t": B.ExpandProblem,
    "dispatch_combine_problem_t": B.CombineProblem,
}


@pytest.mark.parametrize("c_name", sorted(STRUCTS))
def test_struct_layouts_match_the_binding(probe, c_name):
    py = STRUCTS[c_name]
    assert int(probe[f"sizeof.{c_name}"]) == ctypes.sizeof(py)
    c_fields = {k.split(".")[2]: int(v) for k, v in probe.items() if k.startswith(f"offset.{c_name}.")}
    py_fields = {name: getattr(py, name).offset for name, _ in py._fields_}
    assert c_fields == py_fields


def test_versions_match(probe):
    assert int(probe["abi"]) == int(probe["macro_abi"]) == M.dispatch_abi_version() == B.ABI_VERSION


@pytest.mark.parametrize("a", [1, 128])
def test_host_calls_match_the_binding(probe, a):
    p = M.make_problem(4096, 8, 256, 8, a, 8, 14336, 0)
    rc, max_recv, max_rank = (int(v) for v in probe[f"max_rows.a{a}"].split())
    assert rc == 0 and (max_recv, max_rank) == M.dispatch_max_rows(p)
    assert (max_recv, max_rank) == (4096 * 8 + 256 * (a - 1), 4096 * 8)
    rc, ws = (int(v) for v in probe[f"workspace.a{a}"].split())
    assert rc == 0 and ws == M.dispatch_workspace_size(p)
    rc, lay_k, both_k = (int(v) for v in probe[f"kernels.a{a}"].split())
    assert rc == 0 and (lay_k, both_k) == M.dispatch_kernel_count(p)


def test_host_error_from_c(probe):
    assert int(probe["bad_workspace"]) == M.ERR_ARG
    assert probe["strerror_arg"] == M.dispatch_strerror(M.ERR_ARG)
