"""The C ABI used from a plain C program (tests/c_abi_demo.c, built by the
library build next to its source): no Python or torch between the caller and
libblasst.so."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "tests", "c_abi_demo")


def _run(mode):
    assert os.path.exists(DEMO), "tests/c_abi_demo is missing: run the build (__graft_entry__.build()) first"
    r = subprocess.run([DEMO, mode], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr
    return r.stdout


def test_c_program_host_calls():
    """Version, status strings, calibration, the decode planner and argument
    rejection, from C."""
    if not os.path.exists(DEMO):
        from long_context_fa_amd import build
        build.build_c_demo()
    assert "host: ok" in _run("host")


@pytest.mark.gpu
def test_c_program_prefill_on_gpu():
    """A causal prefill from C: at lambda = 0 O equals dense causal softmax
    attention computed by the program; at lambda = 0.3 the skip map holds only
    0, 1 and 255."""
    assert "gpu: ok" in _run("gpu")
