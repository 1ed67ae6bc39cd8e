"""Build libmoe.so (the HIP kernels and the C ABI of include/moe.h) for gfx950.

Every call recompiles: each ``csrc/*.hip`` file becomes an object under
``_build/`` (in parallel), and the objects are linked into ``libmoe.so`` next
to this file.  No GPU is needed to build.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _hipcc():
    return os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    cmd = [_hipcc(), "-c", src, "-o", obj] + CFLAGS
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s" % (src, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# host-side AddressSanitizer + UndefinedBehaviorSanitizer for api.hip (argument
# checks, workspace layouts, launch sequences); -Xarch_host keeps the device code
# uninstrumented
HOST_SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all"


def asan_runtime() -> str:
    """clang's AddressSanitizer runtime (it carries the UBSan handlers too); a
    process loading the sanitized library preloads it."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's AddressSanitizer runtime is not installed")
    return found[-1]


def build_host_sanitized(out: str) -> str:
    """A copy of libmoe.so at ``out`` whose host code in api.hip is built with
    AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts); the
    other translation units are the regular objects.  Load it with
    MOE_LIB_PATH=out and asan_runtime() preloaded."""
    api = os.path.join(CSRC, "api.hip")
    others = [os.path.join(BUILD, os.path.basename(p).replace(".hip", ".o"))
              for p in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) if p != api]
    if not all(os.path.exists(o) for o in others):
        build()
    obj = out + ".api.o"
    flags = [f.replace("-O3", "-O1") for f in CFLAGS] + ["-g", "-fno-omit-frame-pointer"] + HOST_SANITIZE.split()
    r = subprocess.run([_hipcc(), "-c", api, "-o", obj] + flags, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized api.hip:\n%s" % r.stderr)
    r = subprocess.run([_hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", out, obj] + others,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s" % r.stderr)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
