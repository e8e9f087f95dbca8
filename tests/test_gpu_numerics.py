"""Device scalar primitives (exp_f, log_f, BF16 rounding) against the oracle, bitwise,
over their whole binary32 domains."""
import numpy as np
import pytest

from gpu_util import assert_bitwise, f32, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

STEP = 1 << 26


def sweep(orc, fn, lo_bits, hi_bits, ref):
    import invariant_numerics_amd as inv
    for a in range(lo_bits, hi_bits + 1, STEP):
        b = min(hi_bits + 1, a + STEP)
        x = np.arange(a, b, dtype=np.uint64).astype(np.uint32).view(np.float32)
        y = host(inv.inv_eval_numerics(fn, f32(x)))
        assert_bitwise(y, ref(x), "fn %d at 0x%08x" % (fn, a))


def test_exp_f_whole_domain(orc):
    say("exp_f sweep")
    sweep(orc, 0, 0x00000000, 0x42B17218, orc.exp_f)
    sweep(orc, 0, 0x80000000, 0xC2AEAC51, orc.exp_f)


def test_log_f_whole_domain(orc):
    say("log_f sweep")
    sweep(orc, 1, 0x00000001, 0x7F800000, orc.log_f)


def test_bf16_rounding_all_patterns(orc):
    say("bf16 sweep")
    sweep(orc, 2, 0x00000000, 0xFFFFFFFF, lambda x: orc.bf16_up(orc.bf16_rne(x)))
