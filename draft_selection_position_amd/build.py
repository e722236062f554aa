"""Builds libdfs.so (the selector's HIP library for gfx950) in place with hipcc.

Run ``python -m draft_selection_position_amd.build``.  Objects go to ``_build/``
at the repository root; the shared library lands next to this file.  With
``--host-sanitized`` it builds instead ``_build/san/libdfs.so``, whose host code runs under
AddressSanitizer and UBSan (for the C ABI's tests on the CPU).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdfs.so")
SOURCES = ["topk.hip", "gate.hip", "select.hip", "verify.hip", "conv.hip", "lmhead.hip", "static_scratch.hip",
           "dfs_api.cpp"]
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the selector's HIP library cannot be built")


# The host-sanitized build: host code under AddressSanitizer and UBSan (each flag bound to the
# host side), device code as usual.  Its objects and library live under _build/san/.
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libdfs.so")
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), f"--offload-arch={ARCH}", *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libdfs.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def sanitizer_runtime() -> str:
    """The compiler's shared AddressSanitizer runtime (it carries UBSan's handlers too); a
    process that loads the host-sanitized library must preload it."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for base in (os.path.join(root, "llvm", "lib", "clang"), os.path.join(root, "lib", "llvm", "lib", "clang")):
        for ver in sorted(os.listdir(base), reverse=True) if os.path.isdir(base) else []:
            cand = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(cand):
                return cand
    raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")


def build_host_sanitized(verbose: bool = False) -> str:
    """Compile every source with the host code under AddressSanitizer and UBSan (device code
    at -O1: this build is for tests of the host logic on the CPU) and link _build/san/libdfs.so.
    Load it with sanitizer_runtime() preloaded and DFS_LIBRARY naming it."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    extra = [*HOST_SANITIZE, "-O1", "-g"]
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, SAN_BUILD, extra), SOURCES))
    # the sanitizer symbols stay undefined in the library; the preloaded runtime provides them
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv[1:]:
        build_host_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
