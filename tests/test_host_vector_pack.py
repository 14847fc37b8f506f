"""The packed input of the device vector phase, checked on the host.

A compression's Rayleigh-Ritz eigenvectors are formed on the GPU from what the host packs:
the QR iteration's rotation log as runs, groups of runs, (c, s) pairs, plus the reflector
blocks and the wanted positions.  `tests/c/ritz_pack_check.cpp` packs them with the library's
host code and applies them the way the rotation kernel and the reflector products do (same
grouping, wavefront schedule, identity padding and chunking, every row and LDS index checked
against its bounds), then compares with the host eigensolver's own vectors.  The kernel's
constants are read from its source so that the two stay in step.  The GPU kernel itself is
covered by the compression parity tests.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_cross_amd", "csrc")


def kernel_constants():
    src = open(os.path.join(CSRC, "subspace.hip")).read()
    out = {}
    for name, key in [("kRunCap", "KRUNCAP"), ("kB", "KB"), ("CH", "KCH"), ("kSpread", "KSPREAD"),
                      ("kGroupOverhead", "KOVERHEAD")]:
        m = re.search(r"constexpr int %s = (\d+);" % name, src)
        assert m, name
        out[key] = int(m.group(1))
    # the scratch padding the kernel allocates must be what the schedule needs
    assert re.search(r"constexpr int kPadLo = 2 \* CH \+ kB, kPadHi = kB;", src)
    return out


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not shutil.which("g++") or not shutil.which("gcc"):
        pytest.skip("no host C/C++ compiler")
    d = tmp_path_factory.mktemp("ritzpack")
    obj = str(d / "host_eigh.o")
    subprocess.run(["gcc", "-O2", "-march=x86-64-v3", "-std=c11", "-c", os.path.join(CSRC, "host_eigh.c"), "-o", obj],
                   check=True)
    exe = str(d / "ritz_pack_check")
    defs = ["-D%s=%d" % kv for kv in kernel_constants().items()]
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", *defs, "-I", CSRC,
                    os.path.join(ROOT, "tests", "c", "ritz_pack_check.cpp"), obj, "-o", exe], check=True)
    return exe


@pytest.mark.parametrize("args", [
    ("3", "2", "-0.8"),                     # one QR sweep group, no reflector block beyond the first
    ("5", "5", "0.0"),                      # every vector, a flat spectrum
    ("37", "20", "-0.8"),                   # ragged reflector block, r not a multiple of 64
    ("200", "100", "-0.8"),
    ("300", "64", "-0.8", "100", "8"),      # sweeps cut at 100 rotations, groups limited to 8 rows of spread
    ("768", "512", "-1.2"),                 # the 64k workload's Rayleigh-Ritz size
    ("1100", "40", "-1.0"),                 # sweeps longer than the kernel's run cap
    # the log in pieces (piece 0 on the wanted unit vectors, the others on the identity, multiplied)
    ("768", "512", "-1.2", "1024", "64", "4"),   # the 64k workload's Rayleigh-Ritz size, as compressed
    ("1100", "40", "-1.0", "1024", "64", "2"),   # above k_b = 1024: two pieces
    ("300", "64", "-0.8", "100", "8", "4"),      # short runs, narrow groups
    ("37", "20", "-0.8", "1024", "64", "4"),     # few groups
    ("3", "2", "-0.8", "1024", "64", "4"),       # one group: three empty pieces
])
def test_packed_vector_phase_reproduces_host_vectors(checker, args):
    p = subprocess.run([checker, *args], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=300)
    assert p.returncode == 0, p.stdout
    assert "maxdiff" in p.stdout
