"""The host side of the C ABI under AddressSanitizer (CPU only, no GPU needed).

libmol's host code (argument checks, sizing, launch set-up in abi.hip) is rebuilt with the
sanitizer on the host compilation only (device code is untouched), linked with the library's
other objects into a separate shared library, and tests/test_abi.py runs against it in a
child process with the sanitizer runtime preloaded (python itself is not instrumented). Every
error path and sizing helper of the ABI then runs with its memory accesses checked.
"""
import glob
import os
import subprocess
import sys

import pytest

from virtual_expert_routed_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _object(src):
    """The library build's object of src, compiled again if missing or older than a source."""
    obj = os.path.join(build.BUILD, os.path.basename(src) + ".o")
    newest = max(os.path.getmtime(p) for p in glob.glob(os.path.join(build.CSRC, "*")) +
                 glob.glob(os.path.join(ROOT, "include", "*.h")))
    if not os.path.exists(obj) or os.path.getmtime(obj) < newest:
        os.makedirs(build.BUILD, exist_ok=True)
        build._compile(src)
    return obj


def test_abi_tests_pass_with_host_address_sanitizer(tmp_path):
    rt = _runtime()
    if rt is None or not os.path.exists(build.HIPCC):
        pytest.skip("hipcc or the clang AddressSanitizer runtime is not installed")
    abi = os.path.join(build.CSRC, "abi.hip")
    asan_obj = str(tmp_path / "abi_asan.o")
    # the sanitizer flags go to the host compilation only
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in build.CFLAGS if f != "-O3"] + ["-O1"]
    r = subprocess.run([build.HIPCC, *flags, *host_asan, "-I", os.path.join(ROOT, "include"),
                        "-c", abi, "-o", asan_obj], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    others = [_object(s) for s in build.sources() if os.path.basename(s) != "abi.hip"]
    lib = str(tmp_path / "libmol_asan.so")
    r = subprocess.run([build.HIPCC, "-shared", "-fPIC", f"--offload-arch={build.ARCH}",
                        "-Xarch_host", "-fsanitize=address", asan_obj, *others, "-o", lib],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "__asan_" in subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout

    env = dict(os.environ)
    env["MOL_LIBRARY"] = lib
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    # python's own allocations are not instrumented; leaks at exit are not what is checked
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu",
                        "-p", "no:cacheprovider", os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout
