"""Host-side launch rules of the scatter, compiled from the library's own
header with the host compiler and run on the CPU (no GPU):

- lds_for_workgroups_per_cu(n), the dynamic LDS a workgroup reserves so that
  at most n of them share a gfx950 CU (160 KiB of LDS): n of them must fit and
  n + 1 must not, and for the bounds the split scatter uses (n <= 8) that
  stays so when the size is rounded up to any allocation step up to 2 KiB;
- read_ahead_fits, the 160 MB limit on token rows and scale factors that the
  layout reads ahead (and above which the scatter ignores the read-ahead hint).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def probe_output(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("probe") / "launch_rule_probe")
    cmd = [gxx, "-std=c++17", "-O1", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "moe_token_dispatch_amd", "csrc"),
           os.path.join(ROOT, "tests", "launch_rule_probe.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([exe], capture_output=True, text=True, check=True).stdout
    return [line.split() for line in out.splitlines()]


def test_lds_reservation_admits_exactly_n_workgroups(probe_output):
    per_cu = int(next(r[1] for r in probe_output if r[0] == "per_cu"))
    assert per_cu == 160 * 1024
    for _, n, b in (r for r in probe_output if r[0] == "lds"):
        n, b = int(n), int(b)
        assert n * b <= per_cu < (n + 1) * b, (n, b)
        if n <= 8:  # the bounds the scatter uses: exact for any allocation step up to 2 KiB
            for step in (256, 512, 1024, 2048):
                up = -(-b // step) * step
                assert n * up <= per_cu < (n + 1) * up, (n, b, step)


def test_read_ahead_limit(probe_output):
    fits = next(r for r in probe_output if r[0] == "fits")
    # 160 MB exactly fits; 160 MB - 64 B of rows with 16 scale factors (64 B) fits; one word more does not.
    assert fits[1:] == ["1", "1", "0"]
