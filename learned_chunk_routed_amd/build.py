"""Build liblcr.so (HIP kernels for gfx950 + the C ABI) in-tree.

Usage: python -m learned_chunk_routed_amd.build [-v] [--sanitized]

Every HIP translation unit is compiled with hipcc for gfx950 only, with
packed-fp32 instructions disabled; the host-only validation unit is compiled
with g++. Objects go to _build/ at the repository root; the shared library is
written next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "liblcr.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = "gfx950"

HIP_SOURCES = ["summary.hip", "score.hip", "attention.hip", "backward.hip", "api.cpp"]
HOST_SOURCES = ["validate.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    "-I", os.path.join(ROOT, "include"),
]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "unknown target feature" not in l
                    and "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs_list.append([HIPCC] + HIP_FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs_list.append(["g++"] + GXX_FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs_list))
    tmp = OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, OUT)
    return OUT


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same sources, for
# the CPU tests of the C ABI (argument validation, planners, workspace sizes). Only the
# host code is instrumented; the GPU code is built as usual and never runs under it.
SAN_BUILD = os.path.join(BUILD, "sanitized")
SAN_OUT = os.path.join(SAN_BUILD, "liblcr_sanitized.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer"]
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/bin/amdclang++")


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (it carries the UBSan handlers too) that a
    process must preload to load the sanitized library."""
    r = subprocess.run([CLANGXX, "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return path


def build_sanitized(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(SAN_BUILD, exist_ok=True)
    flags = [f for f in HIP_FLAGS if f != "-O3"] + ["-O1", "-g"] + SAN_HOST
    jobs_list, objs = [], []
    for src in HIP_SOURCES:
        obj = os.path.join(SAN_BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs_list.append([HIPCC] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(SAN_BUILD, src + ".o")
        jobs_list.append([CLANGXX, "-O1", "-g", "-std=c++17", "-fPIC", "-fsanitize=address,undefined",
                          "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
                          "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs_list))
    tmp = SAN_OUT + ".tmp"
    _run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-shared-libsan"] + SAN_HOST + ["-o", tmp] + objs,
         verbose)
    os.replace(tmp, SAN_OUT)
    return SAN_OUT


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
