"""include/fa.h is a plain C header: a C99 program that includes it builds
with gcc, links against libfa_mi355x.so and gets the documented rejections
(no GPU needed)."""

import os
import shutil
import subprocess

import pytest

from exact_io_aware_35_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

pytestmark = pytest.mark.skipif(
    not os.path.exists(fb.LIB_PATH) or shutil.which("gcc") is None
    or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")),
    reason="needs the built library, gcc and the HIP headers")


def test_c99_program_builds_links_and_runs(tmp_path):
    exe = tmp_path / "abi_smoke"
    libdir = os.path.dirname(fb.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "c", "abi_smoke.c"), "-o", str(exe),
           "-L", libdir, "-lfa_mi355x", "-Wl,-rpath," + libdir]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.splitlines()
    assert lines[0] == "status=1 name=invalid argument detail=q is null"
    assert lines[1] == "status=1 detail=descale_v must be finite and > 0"
    assert lines[2].startswith("workspace=") and int(lines[2].split("=")[1]) > 0
