"""Build libmamba_scan.so (gfx950) in-tree with hipcc.

    python -m selective_state_space_06_amd.build

Every HIP source is compiled for gfx950 only, with packed-fp32 instruction selection
turned off (-Xclang -target-feature -Xclang -packed-fp32-ops): plain fp32 VALU code.
The host pass warns that it does not know that feature; the warning is harmless.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmamba_scan.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["abi.hip", "scan_fwd.hip", "scan_fast.hip", "scan_bwd.hip", "state_update.hip", "conv1d.hip",
           "ssd_scan.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm under /opt/rocm)")


def compile_flags() -> list[str]:
    return ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]


EXAMPLE_SRC = os.path.join(PKG_DIR, "examples", "scan_from_c.c")
EXAMPLE_BIN = os.path.join(PKG_DIR, "examples", "scan_from_c")


def build_example(verbose: bool = False) -> str:
    """Compile the plain-C example against the built library (host code only: gcc and the HIP
    runtime's C API). Returns the executable's path."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [os.environ.get("CC", "gcc"), "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", INCLUDE, EXAMPLE_SRC, "-L", PKG_DIR, "-lmamba_scan",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath,$ORIGIN/..",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", EXAMPLE_BIN]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"compiling the C example failed with exit code {proc.returncode}")
    return EXAMPLE_BIN


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source (in parallel, one object each) and link them into LIB_PATH
    (atomically replaced), then the C example against it. Returns the library's path."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(PKG_DIR, "_build")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *compile_flags(), *(extra or []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            sys.stderr.write(proc.stdout + proc.stderr)
            raise RuntimeError(f"hipcc failed on {src} with exit code {proc.returncode}")
        return obj

    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB_PATH + f".tmp{os.getpid()}"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        sys.stderr.write(proc.stdout + proc.stderr)
        raise RuntimeError(f"linking failed with exit code {proc.returncode}")
    os.replace(tmp, LIB_PATH)
    build_example(verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
