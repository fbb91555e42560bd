"""Build the gfx950 attention library in-tree (exact_io_aware_35_amd/libfa_mi355x.so).

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled (the compiler would otherwise fuse pairs of fp32 operations into
v_pk_* forms). Objects go to _build/ beside the package; the shared library
is linked into the package directory so it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libfa_mi355x.so")
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ["fa_api.cpp", "fa_fwd.hip", "fa_fwd_fp8.hip", "fa_bwd.hip", "fa_noalloc.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall",
          "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(HERE, "csrc")]
DEVICE = ["-x", "hip", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc", "-munsafe-fp-atomics"]
# Per-source extras. MFMA results go to arch VGPRs: the kernels read every
# score accumulator with VALU ops, and the accumulator-register form would add
# a copy per element (the kernels are shaped to fit 256 VGPRs).
EXTRA = {"fa_fwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fa_fwd_fp8.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
         "fa_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src: str) -> str:
    path = os.path.join(HERE, "csrc", src)
    obj = os.path.join(BUILD_DIR, src + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE if src.endswith(".hip") else ["-D__HIP_PLATFORM_AMD__"])
    cmd += EXTRA.get(src, [])
    cmd += ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass does not know the packed-fp32 feature name; that note is harmless.
    err = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err)
    return obj


def device_asm(src: str, out: str) -> str:
    """Compile one HIP source to gfx950 assembly with the library's flags
    (used by the tests that inspect the generated code)."""
    cmd = [HIPCC] + COMMON + DEVICE + EXTRA.get(src, [])
    cmd += ["--cuda-device-only", "-S", os.path.join(HERE, "csrc", src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", LIB_PATH + ".tmp"] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
