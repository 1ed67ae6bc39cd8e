"""Sanitizer tier (CPU only, no GPU call): the oracle and libmoe's host code
built with AddressSanitizer and UndefinedBehaviorSanitizer, each running its
own CPU test file in a child process with the matching sanitizer runtime
preloaded (gcc's for the oracle, clang's for the hipcc-built library).  Any
report aborts the child, so a clean exit means none was raised."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OPTS = dict(ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0:abort_on_error=1",
            UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _child(args, **env):
    e = dict(os.environ, PYTHONPATH=ROOT, **OPTS, **env)
    r = subprocess.run([sys.executable] + args, cwd=ROOT, env=e, capture_output=True, text=True, timeout=900)
    return r.returncode, r.stdout + r.stderr


def _gcc_asan():
    return subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True,
                          check=True).stdout.strip()


def test_oracle_pins_under_sanitizers(tmp_path):
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    rc, out = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_pins.py"],
                     MOE_ORACLE_LIB=lib, LD_PRELOAD=_gcc_asan())
    assert rc == 0 and " passed" in out, out[-4000:]
    # the instrumentation is live: an overrun of the caller's buffer aborts the child
    probe = ("import numpy as np, oracle\n"
             "lib = oracle._load()\n"
             "x = np.zeros((1, 128), np.float32); q = np.zeros((1, 256), np.uint8); s = np.zeros((1, 2), np.float32)\n"
             "lib.oracle_quant_1x128(1, 256, oracle.F32, x.ctypes.data, q.ctypes.data, s.ctypes.data)\n")
    rc, out = _child(["-c", probe], MOE_ORACLE_LIB=lib, LD_PRELOAD=_gcc_asan())
    assert rc != 0 and "heap-buffer-overflow" in out, out[-2000:]


def test_abi_host_code_under_sanitizers(tmp_path):
    from mixture_experts_layer_35_amd import build
    lib = build.build_host_sanitized(str(tmp_path / "libmoe_san.so"))
    env = dict(MOE_LIB_PATH=lib, LD_PRELOAD=build.asan_runtime())
    rc, out = _child(["-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_abi_cpu.py"], **env)
    assert rc == 0 and " passed" in out, out[-4000:]
    probe = ("import mixture_experts_layer_35_amd as m\n"
             "m.lib()\n"
             "print(any(m.LIB_PATH in l for l in open('/proc/self/maps')))\n")
    rc, out = _child(["-c", probe], **env)
    assert rc == 0 and out.strip().endswith("True"), out[-2000:]
