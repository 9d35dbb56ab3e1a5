"""Code-generation guards for the kernels with AGPR-pinned accumulators (the
latent decode kernel; CPU: hipcc cross-compiles).

These kernels keep their O^T accumulator in physical AGPRs and touch them
only from inline asm.  That is sound only while the
compiler itself allocates no AGPR (for a value, a spill or an MFMA it
emits) and the kernel descriptor reserves all 256 AGPRs.  These tests compile
the source to assembly with the library's own flags and check both, so that
a compiler or source change that breaks the assumption fails here rather than
as corrupted output.
"""
import os
import re
import shutil
import subprocess

import pytest

from long_context_fa_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None,
                                reason="hipcc not available")


KERNELS = {"mla.hip": "decode_mla_kernel"}


@pytest.fixture(scope="module", params=sorted(KERNELS))
def kasm(request, tmp_path_factory):
    out = tmp_path_factory.mktemp("asm") / (request.param + ".s")
    cmd = ([B.HIPCC] + B.FLAGS + B.EXTRA.get(request.param, [])
           + ["-S", "--cuda-device-only", os.path.join(B.CSRC, request.param), "-o", str(out)])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return KERNELS[request.param], out.read_text()


def _outside_asm(text):
    keep, inside = [], False
    for line in text.splitlines():
        if ";;#ASMSTART" in line:
            inside = True
        elif ";;#ASMEND" in line:
            inside = False
        elif not inside:
            keep.append(line.split(";")[0])
    return keep


def _functions(text, kname):
    """(mangled name, body) of every instantiation of kernel ``kname``."""
    return re.findall(r"^(_Z\S*" + kname + r"\S*):(.*?)^\.Lfunc_end", text, re.S | re.M)


def _gap_pass(mangled):
    # the fourth template argument (a bool) is the gap pass, which holds no accumulator
    bools = re.findall(r"Lb([01])E", mangled)
    return len(bools) >= 4 and bools[3] == "1"


def test_compiler_emits_no_agpr_access(kasm):
    kname, text = kasm
    agpr = re.compile(r"\ba\[\d|\ba\d+\b|accvgpr")
    funcs = [(n, body) for n, body in _functions(text, kname) if not _gap_pass(n)]
    assert len(funcs) >= 4
    for name, body in funcs:
        bad = [l for l in _outside_asm(body) if agpr.search(l) and not l.strip().startswith(".")]
        assert not bad, f"{name}: compiler-generated AGPR access:\n" + "\n".join(bad[:10])


def test_no_scratch_and_all_agprs_reserved(kasm):
    kname, text = kasm
    kernels = re.findall(r"\.amdhsa_kernel (\S+)(.*?)\.end_amdhsa_kernel", text, re.S)
    mine = [(n, body) for n, body in kernels if kname in n]
    assert len(mine) >= 5
    for name, body in mine:
        f = dict(re.findall(r"\.amdhsa_(\w+) (\d+)", body))
        assert int(f["private_segment_fixed_size"]) == 0, f"{name} spills"
        if not _gap_pass(name):
            assert int(f["next_free_vgpr"]) - int(f["accum_offset"]) >= 256, f"{name} reserves too few AGPRs"
