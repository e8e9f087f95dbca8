"""Host-side checks of libinvnum.so that need no GPU: it loads, exports every symbol the
header declares, reports the same pinned constants as the oracle, and rejects invalid
arguments with the documented status codes before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "invnum.h")


@pytest.fixture(scope="module")
def inv():
    from invariant_numerics_amd import binding
    return binding


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(inv_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol(inv):
    names = declared_functions()
    assert len(names) >= 14
    lib = ctypes.CDLL(inv.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(inv.EXPORTS) == names


def test_constants_match_oracle(inv, orc):
    c = inv.inv_get_constants()
    fc, ic = orc.constants()
    assert [c["ks"], c["chunk"], c["vocab_tile"], c["lanes"]] == list(ic)
    assert np.array_equal(np.array(c["float_consts"], np.float32).view(np.uint32), fc.view(np.uint32))


def test_status_strings(inv):
    for code in range(0, -8, -1):
        assert inv.inv_status_string(code) not in ("", "unknown status")
    assert inv.inv_status_string(-99) == "unknown status"


FAKE = 1 << 20          # aligned non-null address; never dereferenced by a rejected call
MIS = (1 << 20) + 4     # misaligned


def test_gemm_argument_validation(inv):
    L = inv.LIB
    g = L.inv_fixed_order_gemm
    assert g(None, 4, 64, 64, FAKE, 8, 64, None, 0, FAKE, 8, None) == -1
    assert g(FAKE, 0, 64, 64, FAKE, 8, 64, None, 0, FAKE, 8, None) == -2      # M < 1
    assert g(FAKE, 4, 63, 64, FAKE, 8, 64, None, 0, FAKE, 8, None) == -2      # K % 8
    assert g(FAKE, 4, 64, 32, FAKE, 8, 64, None, 0, FAKE, 8, None) == -2      # ldx < K
    assert g(MIS, 4, 64, 64, FAKE, 8, 64, None, 0, FAKE, 8, None) == -3       # misaligned X
    assert g(FAKE, 4, 64, 66, FAKE, 8, 64, None, 0, FAKE, 8, None) == -3      # ldx % 4


def test_gated_gemm_argument_validation(inv):
    L = inv.LIB
    g = L.inv_gated_gemm
    assert g(None, 1, 64, 64, FAKE, 8, 64, FAKE, 4, None) == -1
    assert g(FAKE, 1, 64, 64, FAKE, 7, 64, FAKE, 4, None) == -2       # odd N2
    assert g(FAKE, 1, 64, 64, FAKE, 8, 64, FAKE, 3, None) == -2       # ldh < N2 / 2
    assert g(FAKE, 1, 60, 64, FAKE, 8, 64, FAKE, 4, None) == -2       # K % 8
    assert g(MIS, 1, 64, 64, FAKE, 8, 64, FAKE, 4, None) == -3        # misaligned X


def test_attention_argument_validation(inv):
    L = inv.LIB
    p = L.inv_attention_prefill
    assert p(1, FAKE, FAKE, FAKE, 1, 4, 0, 8, 4, 2, 64, 1.0, FAKE, None) == -6     # D != 128
    assert p(1, FAKE, FAKE, FAKE, 1, 4, 0, 8, 4, 3, 128, 1.0, FAKE, None) == -2    # Hq % Hkv
    assert p(1, FAKE, FAKE, FAKE, 1, 8, 4, 8, 4, 2, 128, 1.0, FAKE, None) == -2    # q_start+Tq > Tmax
    assert p(7, FAKE, FAKE, FAKE, 1, 4, 0, 8, 4, 2, 128, 1.0, FAKE, None) == -4    # dtype
    d = L.inv_attention_decode
    need = inv.inv_attention_decode_workspace_bytes(2, 512, 4, 128)
    assert need == 4 * 2 * 4 * 2 * 130
    assert d(1, FAKE, FAKE, FAKE, FAKE, 2, 512, 4, 2, 128, 1.0, FAKE, FAKE, need - 4, None) == -5
    assert d(1, FAKE, FAKE, FAKE, None, 2, 512, 4, 2, 128, 1.0, FAKE, FAKE, need, None) == -1


def test_lmhead_argument_validation(inv):
    L = inv.LIB
    f = L.inv_lmhead_logprob_top2
    need = inv.inv_lmhead_workspace_bytes(4, 256, 4096)
    assert need >= 4 * (4 * 256 + 4 * 4096)
    args = [FAKE, 4, 256, 256, FAKE, 4096, FAKE, 0.1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None]
    bad_ws = list(args); bad_ws[14] = need - 1
    assert f(*bad_ws) == -5
    bad_v = list(args); bad_v[5] = 1
    assert f(*bad_v) == -2
    bad_null = list(args); bad_null[6] = None
    assert f(*bad_null) == -1


def test_elementwise_argument_validation(inv):
    L = inv.LIB
    assert L.inv_rmsnorm(FAKE, 4, 4100, 4100, FAKE, 1e-5, FAKE, 4100, None) == -2   # H % 8
    assert L.inv_rmsnorm(FAKE, 4, 32768, 32768, FAKE, 1e-5, FAKE, 32768, None) == -6
    assert L.inv_eval_numerics(3, FAKE, FAKE, 4, None) == -4
    assert L.inv_swiglu(FAKE, FAKE, 2, 8, 4, 8, FAKE, 8, None) == -2
