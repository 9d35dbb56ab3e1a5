"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer.

Host code only: the C ABI layer (api.cpp: validation, planning, calibration,
the no-allocation scratch lookup) is rebuilt with both sanitizers on its host
side and linked with the library's own kernel objects, and the oracle
(oracle.c) is rebuilt with both; then the C-ABI and oracle tests run against
those builds in a child process with the sanitizer runtime preloaded.  Any
report fails the test.  GPU code is never instrumented (GPU sanitizers are
not used here)."""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from long_context_fa_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
ASAN_RT = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
KERNEL_OBJS = [os.path.join(B.BUILD_DIR, f) for f in ("prefill.o", "decode.o", "mla.o")]

pytestmark = pytest.mark.skipif(
    not (os.path.exists(B.HIPCC) and os.path.exists(CLANG) and ASAN_RT and all(map(os.path.exists, KERNEL_OBJS))),
    reason="needs hipcc, the ROCm clang sanitizer runtime and the library's kernel objects (run build() first)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stderr[-3000:]


def test_cpu_suite_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    api_o, lib = str(tmp_path / "api.o"), str(tmp_path / "libblasst.so")
    flags = [f for f in B.FLAGS if f not in ("-O3", "-fPIC")]
    _run([B.HIPCC] + flags + ["-O1", "-g", "-fPIC", "-x", "hip", "-c", os.path.join(B.CSRC, "api.cpp"), "-o", api_o,
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"])
    _run([B.HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", api_o] + KERNEL_OBJS + ["-o", lib])
    olib = str(tmp_path / "liboracle.so")
    _run([CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", os.path.join(ROOT, "oracle", "oracle.c"),
          "-o", olib, "-L/opt/rocm/llvm/lib", "-Wl,-rpath,/opt/rocm/llvm/lib", "-lm"])
    env = dict(os.environ, LD_PRELOAD=ASAN_RT[-1], ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", BLASST_LIBRARY=lib, ORACLE_LIB_OVERRIDE=olib,
               OMP_NUM_THREADS="4")
    tests = [os.path.join(ROOT, "tests", f) for f in ("test_abi_cpu.py", "test_oracle_pins.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"] + tests,
                       env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
