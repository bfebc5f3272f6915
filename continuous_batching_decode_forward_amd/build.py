"""Build libcbd.so (the HIP kernels, host runtime and C ABI) for gfx950.

    python -m continuous_batching_decode_forward_amd.build [--force]

Every source in csrc/ is compiled with hipcc for gfx950 only; the shared
library lands next to this file, in-tree. csrc/check/ holds a host-only
replay of the attention schedule (the kernels' own schedule arithmetic from
csrc/attn_sched.h), built into libcbd_schedcheck.so for the tests.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcbd.so")
CHECK_LIB = os.path.join(HERE, "libcbd_schedcheck.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.environ.get("HIPCC", os.path.join(ROCM, "bin", "hipcc"))

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function", f"-I{INCLUDE}"]
# Packed fp32 instructions stay off in device code.
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=fast", "-munsafe-fp-atomics"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    else:  # host-only C++ (the HIP runtime API, no device code)
        cmd += ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{r.stderr}")
    return obj


def check_sources():
    return sorted(glob.glob(os.path.join(CSRC, "check", "*.cpp")))


def _stale() -> bool:
    deps = sources() + check_sources() + glob.glob(os.path.join(CSRC, "*.h")) + \
        [os.path.join(INCLUDE, "cbd.h")]
    for lib in (LIB, CHECK_LIB):
        if not os.path.exists(lib):
            return True
        t = os.path.getmtime(lib)
        if any(os.path.getmtime(p) > t for p in deps):
            return True
    return False


def _build_check() -> None:
    tmp = CHECK_LIB + ".tmp"
    cmd = [HIPCC] + COMMON + ["-x", "c++", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include",
                              "-shared", "-o", tmp] + check_sources()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"schedule checker build failed:\n{r.stderr}")
    os.replace(tmp, CHECK_LIB)


def build(force: bool = False, jobs: int = 8) -> str:
    if not force and not _stale():
        return LIB
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, sources()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    _build_check()
    return LIB


if __name__ == "__main__":
    print(build(force="--force" in sys.argv))
