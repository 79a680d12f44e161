import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def brute_lib(tmp_path_factory):
    """The independent brute-force E4M3 encoder (tests/csrc/brute_e4m3.c)."""
    import ctypes
    src = os.path.join(ROOT, "tests", "csrc", "brute_e4m3.c")
    out = str(tmp_path_factory.mktemp("brute") / "libbrute.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fopenmp", "-fPIC",
                           "-shared", "-o", out, src, "-lm"])
    return ctypes.CDLL(out)
