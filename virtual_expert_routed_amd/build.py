"""Build libmol.so (the HIP kernels and their C ABI) for gfx950, in-tree.

    python -m virtual_expert_routed_amd.build

Compiles every csrc/*.hip with hipcc in parallel, links the shared library next to this
file (and, apart from it, the benchmark's read-only streaming probe libmolcalib.so), then lists the code objects embedded in it and fails unless a gfx950 one is there
(a build that silently drops the target architecture still "succeeds" otherwise).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmol.so")
# the benchmark's read-only streaming probe, a library of its own (not part of libmol)
CALIB_SRC = os.path.join(PKG, "calib", "read_probe.hip")
CALIB_LIB = os.path.join(PKG, "libmolcalib.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # packed fp32 instructions are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first eight kernel parameters arrive preloaded in scalar registers (the delta
    # kernels pass their routing arguments there)
    "-mllvm", "-amdgpu-kernarg-preload-count=8",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def code_objects(path: str = LIB) -> list:
    """Entries of the offload bundle in the library's .hip_fatbin section."""
    fatbin = os.path.join(BUILD, os.path.basename(path) + ".hip_fatbin")
    subprocess.run(["objcopy", "-O", "binary", "--only-section=.hip_fatbin", path, fatbin],
                   check=True)
    r = subprocess.run(["/opt/rocm/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                        f"--input={fatbin}"], capture_output=True, text=True, check=True)
    return [ln.strip() for ln in r.stdout.splitlines() if ln.strip()]


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources() + [CALIB_SRC]
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    calib_obj = objs.pop()
    _link([calib_obj], CALIB_LIB, verbose=False)
    return _link(objs, LIB, verbose)


def _link(objs: list, lib_path: str, verbose: bool) -> str:
    tmp = lib_path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    objs_listed = code_objects(tmp)
    if not any(ARCH in ln for ln in objs_listed):
        raise RuntimeError(f"{tmp} carries no {ARCH} code object: {objs_listed}")
    os.replace(tmp, lib_path)
    if verbose:
        print(f"built {lib_path} ({os.path.getsize(lib_path)} bytes); code objects:")
        for ln in objs_listed:
            print("   ", ln)
    return lib_path


if __name__ == "__main__":
    build()
    sys.exit(0)
