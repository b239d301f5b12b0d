"""Build the csakv HIP library (gfx950) in-tree: ``compressed_sparse_kv_csa_amd/libcsakv.so``.

Every source under ``csrc/`` is compiled by hipcc for gfx950 only, in parallel, and
linked into one shared library with a C ABI (``include/csakv.h``).
Usage: ``python -m compressed_sparse_kv_csa_amd.build [--resource-usage] [--host-sanitize]``.

``--host-sanitize`` (after a normal build) also links ``_build/libcsakv_hostsan.so``: the C
ABI's host code (``capi.cpp``: validation, workspace layout, byte accounting) compiled with
AddressSanitizer and UndefinedBehaviorSanitizer for the host only (``-Xarch_host``), linked
with the unchanged GPU objects.  Load it with the sanitizer runtime preloaded
(``host_sanitizer_runtime()``) and ``CSAKV_LIBRARY`` pointing at it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcsakv.so")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# Per-source extra flags.  attention.hip: MFMA accumulators in VGPRs (the default keeps the
# output accumulators in AGPRs and copies all 32 of them to VGPRs on every iteration of the
# step loop, around the rare rescale).
FILE_FLAGS = {
    "attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


SAN_LIB = os.path.join(BUILD, "libcsakv_hostsan.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]


def host_sanitizer_runtime() -> str:
    """Path of the AddressSanitizer runtime of the compiler that builds the library."""
    import glob
    llvm = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm")
    hits = sorted(glob.glob(os.path.join(llvm, "lib", "clang", "*", "lib", "linux",
                                         "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("no clang AddressSanitizer runtime found next to hipcc")
    return os.path.realpath(hits[-1])


def build_host_sanitized() -> str:
    """Link _build/libcsakv_hostsan.so: capi.cpp with host ASan + UBSan, the other objects as
    built by build()."""
    src = os.path.join(CSRC, "capi.cpp")
    obj = os.path.join(BUILD, "capi.cpp.hostsan.o")
    cmd = [_hipcc(), "-x", "hip", *CFLAGS, *SAN_FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on capi.cpp (host sanitizers):\n{r.stdout}{r.stderr}")
    objs = [os.path.join(BUILD, os.path.basename(x) + ".o") for x in _sources()
            if not x.endswith("capi.cpp")]
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", SAN_LIB,
           obj, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (host sanitizers):\n{r.stdout}{r.stderr}")
    return SAN_LIB


def _hipcc() -> str:
    p = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(p):
        raise RuntimeError("hipcc not found: the csakv library needs ROCm's hipcc to build")
    return p


def _sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str, resource_usage: bool) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if resource_usage:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{log}")
    return obj, log


def build(resource_usage: bool = False, verbose: bool = False) -> str:
    """Compile every source and link ``libcsakv.so``; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = _sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, resource_usage), srcs))
    objs = [o for o, _ in results]
    if verbose or resource_usage:
        for _, log in results:
            if log.strip():
                print(log)
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(resource_usage="--resource-usage" in sys.argv, verbose="-v" in sys.argv))
    if "--host-sanitize" in sys.argv:
        print(build_host_sanitized())
