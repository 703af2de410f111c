"""Builds libkvepi.so in-tree with hipcc for gfx950 (no GPU needed)."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG, "libkvepi.so")
SOURCES = [os.path.join(CSRC, n) for n in ("kvepi_kernels.hip", "kvepi_host.cpp",
                                           "kvepi_debug.cpp", "kvepi_drq.hip",
                                           "kvepi_drq_host.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "-fvisibility=hidden",  # export only the C ABI
    # the epilog's arithmetic is IEEE binary32 in source order
    "-ffp-contract=off", "-fno-fast-math",
    # never let the compiler form packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}")


def build(force: bool = True, verbose: bool = False) -> str:
    """Compiles every source to an object (in parallel), then links."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="kvepi_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.basename(src) + ".o") for src in SOURCES]
        cmds = [[hipcc(), *compile_flags, "-I", INCLUDE, "-I", CSRC, "-c", "-o", obj, src]
                for src, obj in zip(SOURCES, objs)]
        with ThreadPoolExecutor(max_workers=len(cmds)) as pool:
            for f in [pool.submit(_run, c, verbose) for c in cmds]:
                f.result()
        tmp = LIB_PATH + ".tmp"
        _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


CEILING_SRC = os.path.join(CSRC, "kvepi_ceiling.hip")
CEILING_LIB = os.path.join(PKG, "libkvepi_ceiling.so")


def build_ceiling(verbose: bool = False) -> str:
    """Builds libkvepi_ceiling.so, the reference memory kernels bench.py
    times beside the epilog (a separate library: not part of the C ABI)."""
    tmp = CEILING_LIB + ".tmp"
    _run([hipcc(), *HIPCC_FLAGS, "-o", tmp, CEILING_SRC], verbose)
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


HW_CHECK_SRC = os.path.join(ROOT, "tests", "hw_check.hip")
HW_CHECK_BIN = os.path.join(ROOT, "tests", "hw_check")


def build_hw_check(verbose: bool = False) -> str:
    """Builds tests/hw_check, the GPU check of the hardware instructions the
    kernels rely on (run by a GPU test; a separate program, not linked into
    the library)."""
    tmp = HW_CHECK_BIN + ".tmp"
    flags = [f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared", "-fvisibility=hidden")]
    cmd = [hipcc(), *flags, "-I", CSRC, "-o", tmp, HW_CHECK_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}")
    os.replace(tmp, HW_CHECK_BIN)
    return HW_CHECK_BIN


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c_client.c")
C_CLIENT_BIN = os.path.join(ROOT, "tests", "c_client")


def build_c_client(verbose: bool = False) -> str:
    """Builds tests/c_client, a plain C11 program (gcc, no C++) that drives
    the epilog through include/kvepi.h and the HIP runtime's C API only,
    linked against the in-tree libkvepi.so (run by a GPU test)."""
    tmp = C_CLIENT_BIN + ".tmp"
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", INCLUDE, "-I", os.path.join(rocm, "include"), "-o", tmp, C_CLIENT_SRC,
           "-L", PKG, "-lkvepi", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../kv_cache_epilog_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    _run(cmd, verbose)
    os.replace(tmp, C_CLIENT_BIN)
    return C_CLIENT_BIN


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_ceiling(verbose=True))
    print(build_hw_check(verbose=True))
    print(build_c_client(verbose=True))
