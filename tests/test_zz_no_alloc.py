"""The allocation-free decode entry point (inv_attention_decode_noalloc, for callers that cannot
allocate) against inv_attention_decode with a caller workspace: bitwise equal, on two calls in
a row, the second with fewer rows and a shorter cache, so the shared scratch array keeps the
first call's partials while the second runs."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitwise, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

D = 128


def inv():
    import invariant_numerics_amd as m
    return m


def case(seed, B, Hq, Hkv, T, pos, bf):
    q = synth.normal(seed, (B, Hq, D))
    k = synth.normal(seed + 1, (B, Hkv, T, D))
    v = synth.normal(seed + 2, (B, Hkv, T, D))
    if bf:
        q, k, v = (torch.from_numpy(synth.to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
                   for a in (q, k, v))
    else:
        q, k, v = (torch.from_numpy(a).cuda() for a in (q, k, v))
    return q, k, v, torch.tensor(pos, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("bf", [False, True])
def test_noalloc_decode_equals_workspace_decode(bf):
    calls = [(14100, 4, 32, 8, 32768, [32767, 20000, 256, 0]),     # large first call
             (14200, 2, 8, 2, 3000, [2999, 511])]                   # smaller second call
    outs = []
    for seed, B, Hq, Hkv, T, pos in calls:
        say("noalloc decode", B, Hq, Hkv, T, bf)
        q, k, v, p = case(seed, B, Hq, Hkv, T, pos, bf)
        assert inv().inv_attention_decode_workspace_bytes(B, T, Hq, D) <= inv().inv_attention_decode_noalloc_max_bytes()
        want = host(inv().inv_attention_decode(q, k, v, p))
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        got = host(inv().inv_attention_decode_noalloc(q, k, v, p, out))
        assert_bitwise(got, want, "noalloc B=%d T=%d" % (B, T))
        outs.append(got)
    # the first call's result is unchanged by the second (outputs are the caller's)
    assert np.isfinite(outs[0]).all() and np.isfinite(outs[1]).all()


def test_noalloc_decode_rejects_oversized():
    """16 rows of 32 heads at a 32k cache need more than the fixed array: rejected before any
    launch (the tensors' contents are never read)."""
    q = torch.empty((16, 32, D), dtype=torch.float32, device="cuda")
    k = torch.empty((16, 8, 32768, D), dtype=torch.float32, device="cuda")
    p = torch.full((16,), 100, dtype=torch.int32, device="cuda")
    out = torch.empty((16, 32, D), dtype=torch.float32, device="cuda")
    v = k
    with pytest.raises(inv().InvError):
        inv().inv_attention_decode_noalloc(q, k, v, p, out)
