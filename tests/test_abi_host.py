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


def test_rmsnorm_fused_argument_validation(inv):
    L = inv.LIB
    g = L.inv_rmsnorm_gemm
    OUT = FAKE + (1 << 20)                    # an output 1 MiB away from X
    assert g(None, 1, 64, 64, FAKE, 1e-5, FAKE, 8, 64, None, 0, OUT, 8, 0, None) == -1
    assert g(FAKE, 1, 64, 64, None, 1e-5, FAKE, 8, 64, None, 0, OUT, 8, 0, None) == -1    # no gains
    assert g(FAKE, 1, 64, 64, FAKE, 1e-5, FAKE, 8, 64, None, 0, OUT, 8, 2, None) == -2    # gated not 0/1
    assert g(FAKE, 1, 64, 64, FAKE, 1e-5, FAKE, 7, 64, None, 0, OUT, 8, 1, None) == -2    # gated, odd N
    assert g(FAKE, 1, 64, 64, FAKE, 1e-5, FAKE, 8, 64, FAKE, 8, OUT, 8, 1, None) == -2    # gated with R
    assert g(FAKE, 1, 60, 64, FAKE, 1e-5, FAKE, 8, 64, None, 0, OUT, 8, 0, None) == -2    # K % 8
    assert g(FAKE, 5, 64, 64, FAKE, 1e-5, FAKE, 8, 64, None, 0, OUT, 8, 0, None) == -6    # M > 4
    assert g(FAKE, 1, 16392, 16392, FAKE, 1e-5, FAKE, 8, 16392, None, 0, OUT, 8, 0, None) == -6  # K > 16384
    assert g(FAKE, 1, 64, 64, MIS, 1e-5, FAKE, 8, 64, None, 0, OUT, 8, 0, None) == -3     # misaligned gains
    assert g(FAKE, 2, 64, 64, FAKE, 1e-5, FAKE, 8, 64, None, 0, FAKE + 256, 8, 0, None) == -2  # Y overlaps X
    q = L.inv_rmsnorm_qkv_rope_kv_append
    args = [FAKE, 1, 64, 64, FAKE, 1e-5, FAKE, 64, 2, 1, 128, FAKE, FAKE, FAKE, FAKE, 16, 1, OUT, OUT + (1 << 16),
            OUT + (1 << 17), None]
    bad = list(args); bad[4] = None
    assert q(*bad) == -1
    bad = list(args); bad[1] = 5
    assert q(*bad) == -6                                                                # M > 4
    bad = list(args); bad[10] = 64
    assert q(*bad) == -6                                                                # D != 128
    bad = list(args); bad[17] = FAKE
    assert q(*bad) == -2                                                                # Qout overlaps X


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


def test_kernel_route_names(inv):
    """The route query names the instantiation each shape class reaches (the tests that
    compare the benchmarked kernels with the oracle assert their shapes with it)."""
    r = inv.inv_kernel_route
    assert r("gemm", 1, 4096) == "gemm_skinny_kernel<1,0,4>"
    assert r("gemm", 1, 28672) == "gemm_skinny_kernel<1,0,16>"
    assert r("gemm", 3, 4096) == "gemm_skinny_kernel<4,0,16,1>"
    assert r("gemm", 16, 4096) == "gemm_gemv16_kernel<1,2,64,0,1,8>"
    assert r("gemm", 16, 6144) == "gemm_gemv16_kernel<1,2,64,0,1,4>"
    assert r("gemm", 32, 14336) == "gemm_gemv16_kernel<2,2,64,0,2,4>"
    assert r("gemm", 64, 4096) == "gemm_gemv16_kernel<1,2,32,0,2,4> by 32-row groups"
    assert r("gemm", 40, 2048) == "gemm_gemv16_kernel<1,2,64,0,1,4> by 16-row groups"
    assert r("gemm", 24, 6144) == "gemm_gemv16_kernel<1,2,64,0,1,4> by 16-row groups"
    assert r("gemm", 24, 4096) == "gemm_gemv16_kernel<1,2,64,0,2,4>"
    assert r("gemm", 48, 4096) == "gemm_gemv16_kernel<1,2,64,0,1,4> by 16-row groups"
    assert r("gemm", 40, 6144) == "gemm_gemv16_kernel<1,2,64,0,1,4> by 16-row groups"
    assert r("gemm", 64, 8192) == "gemm_gemv16_kernel<1,2,32,0,2,4> by 32-row groups"
    assert not r("gemm", 64, 14336).startswith("gemm_gemv16")
    assert r("gemm", 64, 16384) == "gemm_mfma_kernel<64,64,2,2,0>"
    assert r("gemm", 512, 4096) == "gemm_mfma_kernel<64,128,2,4,0>"
    assert r("gemm", 1024, 14336) == "gemm_mfma_kernel<64,128,2,4,0>"
    assert r("gemm", 512, 14336) == "gemm_mfma_kernel<64,64,2,2,0>"
    assert r("gemm", 2048, 4096) == "gemm_mfma_kernel<128,256,2,4,0>"
    assert r("lmhead_gemm", 128, 128256) == "gemm_mfma_kernel<128,256,2,4,1>"
    assert r("gemm", 257, 4096) == "gemm_mfma_kernel<64,64,2,2,0>+gemm_skinny_kernel<1,0,4>"
    assert r("gemm", 256, 4096) == "gemm_mfma_kernel<64,64,2,2,0>"
    assert r("gemm", 260, 9000) == "gemm_mfma_kernel<64,128,2,4,0>+gemm_skinny_kernel<4,0,16,1>"
    assert r("gemm", 128, 4096) == "gemm_small_kernel<0>"
    assert r("gemm", 257, 14336) == "gemm_mfma_kernel<64,128,2,4,0>+gemm_skinny_kernel<1,0,4>"
    assert r("gemm", 1024, 8192) == "gemm_mfma_kernel<128,256,2,4,0>"
    assert r("gemm", 16384, 6144) == "gemm_mfma_kernel<128,256,2,4,0>"
    assert r("gated_gemm", 1024, 8192) == "gemm_mfma_kernel<128,256,2,4,2>"
    assert r("gated_gemm", 1, 28672) == "gemm_skinny_kernel<1,2,16>"
    assert r("lmhead_gemm", 1, 128256) == "gemm_skinny_kernel<2,1,16>"
    assert r("lmhead_gemm", 8, 128256) == "gemm_gemv16_kernel<4,2,64,1,1,8>"
    assert r("lmhead_gemm", 32, 128256) == "gemm_mfma_kernel<64,64,2,2,1>"     # 64 rows, one sweep
    assert r("lmhead_gemm", 32767, 128256) == "gemm_mfma_kernel<128,256,2,4,1>"
    assert r("attention_prefill", 4 * 32, 512) == "attn_prefill_kernel<DT,8,64>"
    assert r("attention_prefill", 8, 2048) == "attn_prefill_kernel<DT,4,32>"
    assert inv.LIB.inv_kernel_route(9, 1, 1, ctypes.create_string_buffer(8), 8) == -4
    assert inv.LIB.inv_kernel_route(0, 0, 1, ctypes.create_string_buffer(8), 8) == -2
    assert inv.LIB.inv_kernel_route(0, 1, 1, None, 8) == -1


def test_decode_noalloc_rejects_oversized_calls(inv):
    """The allocation-free decode checks its size against the library's fixed array before
    anything else: too many rows for the array is INV_ERR_WORKSPACE, nothing launched."""
    L = inv.LIB
    cap = inv.inv_attention_decode_noalloc_max_bytes()
    assert cap == 32 << 20
    per_row = inv.inv_attention_decode_workspace_bytes(1, 32768, 32, 128)
    assert per_row * 15 <= cap < per_row * 16
    f = L.inv_attention_decode_noalloc
    assert f(1, FAKE, FAKE, FAKE, FAKE, 16, 32768, 32, 8, 128, 1.0, FAKE, None) == -5
    assert f(1, FAKE, FAKE, FAKE, None, 1, 32768, 32, 8, 128, 1.0, FAKE, None) == -1
    assert f(1, FAKE, FAKE, FAKE, FAKE, 1, 32768, 32, 8, 64, 1.0, FAKE, None) == -6


def test_probe_argument_validation(inv):
    """The two measurement probes validate their arguments before launching anything."""
    L = inv.LIB
    assert L.inv_read_stream_probe(None, 1024, FAKE, 64, None) == -1
    assert L.inv_read_stream_probe(FAKE, 1000, FAKE, 64, None) == -2      # not a multiple of 16
    assert L.inv_read_stream_probe(FAKE, 1024, FAKE, 0, None) == -2
    assert L.inv_mfma_rate_probe(2, 10, 8, FAKE, None) == -4              # no such instruction
    assert L.inv_mfma_rate_probe(0, 10, 6, FAKE, None) == -2              # not a multiple of 4
    assert L.inv_mfma_rate_probe(1, 0, 8, FAKE, None) == -2
    assert L.inv_mfma_rate_probe(1, 10, 8, None, None) == -1
