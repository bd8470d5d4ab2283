"""Checks on the gfx950 assembly the HIP sources compile to (CPU only).

The LDS-staged kernels (the sketch contractions and the apply sweeps) issue
their global-to-LDS copies from inline asm, where the compiler cannot insert
the wait states the hardware needs before a vector-memory instruction whose
scalar base (or M0) was just written. The asm therefore starts each copy
with s_nop 4; this test compiles those sources to device assembly and checks
that every copy in every kernel has those five wait states in front of it.
"""
import os
import re
import shutil
import subprocess

import pytest

from rank_randomized_gradient_amd import build

STAGED_SOURCES = ["rgc_sketch.hip", "rgc_apply.hip"]


@pytest.fixture(scope="module", params=STAGED_SOURCES)
def staged_asm(request, tmp_path_factory):
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / (request.param + ".s")
    flags = [f for f in build.HIP_FLAGS if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
    cmd = [cc, *flags, "--cuda-device-only", "-S", os.path.join(build.CSRC, request.param), "-o", str(out)]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-2000:]
    return out.read_text()


def _instructions(text):
    """(kernel, instruction) pairs in order, without labels, comments and directives."""
    kernel = None
    for line in text.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            kernel = m.group(1)
            continue
        s = line.strip()
        if not s or s.startswith((";", ".")) or s.endswith(":"):
            continue
        yield kernel, s


def test_every_lds_copy_has_five_wait_states(staged_asm):
    prev = []
    copies = 0
    for kernel, inst in _instructions(staged_asm):
        if inst.startswith("global_load_lds"):
            copies += 1
            assert prev and prev[-1] == "s_nop 4", f"{kernel}: {inst} follows {prev[-1] if prev else None}"
        prev.append(inst)
    assert copies > 0, "no global-to-LDS copies found"
