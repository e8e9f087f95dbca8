import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: long CPU-only check")


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as o
    o.lib()
    return o


@pytest.fixture(scope="session")
def numcheck(tmp_path_factory, orc):
    """Exhaustive primitive checker (tests/csrc/numerics_check.c) linked to the oracle."""
    import ctypes
    out = tmp_path_factory.mktemp("numcheck") / "libnumcheck.so"
    odir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(out),
                    os.path.join(TESTS, "csrc", "numerics_check.c"), "-L", odir, "-loracle",
                    "-Wl,-rpath," + odir, "-lm"], check=True)
    L = ctypes.CDLL(str(out))
    L.max_ulp_err.restype = ctypes.c_double
    L.max_ulp_err.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint32,
                              ctypes.POINTER(ctypes.c_uint32)]
    L.check_bf16_range.restype = ctypes.c_uint64
    L.check_bf16_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.check_f16_range.restype = ctypes.c_uint64
    L.check_f16_range.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
    L.check_f16_up.restype = ctypes.c_uint64
    L.check_f16_up.argtypes = []
    return L
