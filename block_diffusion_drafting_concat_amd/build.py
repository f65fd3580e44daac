"""Build libdflash.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Every call recompiles. `python -m block_diffusion_drafting_concat_amd.build` does the same
from the command line."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libdflash.so")
SOURCES = ["api.cpp", "profile.cpp", "gemm.hip", "attention.hip", "rowwise.hip", "persist.hip"]
ARCH = "gfx950"
# Packed fp32 VALU instructions are kept out of every kernel (hipcc would otherwise form them
# from plain float code).
FLAGS = ["-x", "hip", f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    # -z defs: a kernel whose host stub was not emitted fails the link instead of the launch
    r = subprocess.run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-only AddressSanitizer: every -fsanitize flag goes to the host compilation (-Xarch_host),
# so the GPU code objects are built as usual.
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_DRIVER = os.path.join(BUILD, "abi_asan")


def build_asan_driver() -> str:
    """Build the host ABI checks (tests/abi_asan_main.cpp) against api.cpp and profile.cpp
    compiled with host-only AddressSanitizer and the regular kernel objects. Returns the path
    of the executable."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    kern = [os.path.join(BUILD, n) for n in ("gemm.o", "attention.o", "rowwise.o", "persist.o")]
    if not all(os.path.exists(k) for k in kern):
        build()
    srcs = [os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "profile.cpp"),
            os.path.join(ROOT, "tests", "abi_asan_main.cpp")]

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, "asan_" + os.path.splitext(os.path.basename(src))[0] + ".o")
        r = subprocess.run([cc, *FLAGS, "-O1", *ASAN_HOST, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(compile_one, srcs))
    r = subprocess.run([cc, f"--offload-arch={ARCH}", *ASAN_HOST, "-o", ASAN_DRIVER, *objs, *kern],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    return ASAN_DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
