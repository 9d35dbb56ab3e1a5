"""Build libblasst.so (HIP kernels for gfx950 + the C ABI) in-tree.

    python -m long_context_fa_amd.build      # or: python long_context_fa_amd/build.py

Every HIP source is compiled for gfx950 only, with packed-fp32 code
generation disabled, then linked into long_context_fa_amd/libblasst.so.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "libblasst.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["api.cpp", "prefill.hip", "decode.hip", "mla.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]
# Per source: the GQA decode kernel runs one wave per SIMD; without this the
# compiler keeps its P.V accumulators in AGPRs and copies them to VGPRs and
# back on every block.
EXTRA = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _compile(src, verbose):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err)
    return obj


DEMO_SRC = os.path.join(ROOT, "tests", "c_abi_demo.c")
DEMO_OUT = os.path.join(ROOT, "tests", "c_abi_demo")


def build_c_demo(verbose=False):
    """The plain-C program of the tests that calls libblasst.so through the C
    ABI alone (no Python, no torch); built next to its source."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", "/opt/rocm/include",
           DEMO_SRC, "-L", HERE, "-lblasst", "-L", "/opt/rocm/lib", "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../long_context_fa_amd", "-Wl,-rpath,/opt/rocm/lib", "-o", DEMO_OUT]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return DEMO_OUT


def build(verbose=False):
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    build_c_demo(verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
