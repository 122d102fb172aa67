"""Compile the HIP library libduolm.so for gfx950 in-tree.

Every source is compiled with hipcc (one object each, in parallel) and linked
into ``shared_prefix_scoring_amd/lib/libduolm.so``.  Packed-fp32 instructions
are disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libduolm.so")

SOURCES = ["api.cpp", "k_elem.hip", "k_gemm.hip", "k_attn.hip", "k_export.hip"]
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every multiply-add is written out (fmaf where fused): the compiler may not
    # contract differently in different kernel instantiations, which keeps
    # results independent of tile shape and batch composition
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm install missing)")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


ASAN_PATH = os.path.join(LIB_DIR, "duolm_host_asan")
ASAN_DRIVER = os.path.join(os.path.dirname(PKG), "tests", "asan", "host_asan.cpp")
# AddressSanitizer on host code only (device code is built as usual)
ASAN_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def _run(cmd, what):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        errs = "\n".join(l for l in r.stderr.splitlines() if "not a recognized feature" not in l)
        raise RuntimeError(f"{what} failed:\n{errs}")


def build_host_asan(objs) -> str:
    """The host-sanitizer test driver (tests/asan/host_asan.cpp), linked with
    api.cpp built with ASAN_HOST and the device objects as they are."""
    api = os.path.join(BUILD_DIR, "api_asan.o")
    drv = os.path.join(BUILD_DIR, "host_asan.o")
    _run([hipcc(), *FLAGS, *ASAN_HOST, "-x", "hip", "-c", os.path.join(CSRC, "api.cpp"), "-o", api], "api.cpp (asan)")
    _run([hipcc(), "-O1", "-std=c++17", *ASAN_HOST, "-I", os.path.join(os.path.dirname(PKG), "include"), "-x", "c++",
          "-c", ASAN_DRIVER, "-o", drv], "host_asan.cpp")
    dev = [o for o in objs if not o.endswith("api.o")]
    tmp = ASAN_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", *ASAN_HOST, drv, api, *dev, "-o", tmp], "host_asan link")
    os.replace(tmp, ASAN_PATH)
    return ASAN_PATH


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB_PATH)
    if os.path.exists(ASAN_DRIVER):
        # test tooling: a toolchain without the sanitizer runtime still builds the library
        try:
            build_host_asan(objs)
        except RuntimeError as e:
            sys.stderr.write(f"warning: host-sanitizer test driver not built: {e}\n")
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
