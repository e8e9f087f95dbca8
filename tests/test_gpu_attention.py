"""attention_prefill / attention_decode on the GPU: bitwise equal to the oracle, and the
prefill row equals the token-by-token decode row (fixed 256-key chunks, one merge order)."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

D = 128


def inv():
    import invariant_numerics_amd as m
    return m


def rand_qkv(seed, B, T, Hq, Hkv, bf=False):
    q = synth.normal(seed, (B, T, Hq, D))
    k = synth.normal(seed + 1, (B, Hkv, T, D))
    v = synth.normal(seed + 2, (B, Hkv, T, D))
    if bf:
        return synth.to_bf16_bits(q), synth.to_bf16_bits(k), synth.to_bf16_bits(v)
    return q, k, v


def dev(a):
    return bf16(a) if a.dtype == np.uint16 else f32(a)


@pytest.mark.parametrize("B,T,Hq,Hkv,bf", [(1, 1, 1, 1, False), (1, 70, 2, 2, False), (2, 300, 4, 2, False),
                                           (1, 530, 4, 1, True), (1, 777, 8, 2, False)])
def test_prefill_matches_oracle(orc, B, T, Hq, Hkv, bf):
    say("attn prefill", B, T, Hq, Hkv, bf)
    q, k, v = rand_qkv(8000 + T, B, T, Hq, Hkv, bf)
    O = host(inv().inv_attention_prefill(dev(q), dev(k), dev(v)))
    assert_bitwise(O, orc.attention(q, k, v), "prefill")


def test_prefill_query_blocks_and_offsets(orc):
    """Queries at an offset (q_start, not a multiple of 64) give the same rows."""
    say("attn q_start")
    q, k, v = rand_qkv(8100, 2, 600, 4, 2)
    full = host(inv().inv_attention_prefill(f32(q), f32(k), f32(v)))
    for s in (1, 200, 255, 256, 300, 599):
        part = host(inv().inv_attention_prefill(f32(q[:, s:].copy()), f32(k), f32(v), q_start=s))
        assert_bitwise(part, full[:, s:], "q_start=%d" % s)


def test_decode_matches_prefill_rows_ragged_positions(orc):
    say("attn decode ragged")
    B, T, Hq, Hkv = 3, 700, 8, 2
    q, k, v = rand_qkv(8200, B, T, Hq, Hkv)
    full = host(inv().inv_attention_prefill(f32(q), f32(k), f32(v)))
    kd, vd = f32(k), f32(v)
    for posv in ([0, 255, 256], [511, 512, 699], [100, 600, 300]):
        pos = np.array(posv, np.int32)
        qd = np.stack([q[b, pos[b]] for b in range(B)])
        O = host(inv().inv_attention_decode(f32(qd), kd, vd, i32(pos)))
        want = np.stack([full[b, pos[b]] for b in range(B)])
        assert_bitwise(O, want, "decode pos=%s" % posv)


@pytest.mark.parametrize("bf", [False, True])
def test_large_grid_prefill_equals_decode_and_small_grid(bf):
    """A prefill big enough for the 128-row workgroups (32 heads x 2048 rows) equals decode at
    sampled positions and, row for row, the same queries run as small calls (one 16-row block
    of 4 heads at a time, 64-row workgroups): the workgroup size never changes a bit."""
    say("attn large grid", bf)
    B, T, Hq, Hkv = 1, 2048, 32, 8
    q, k, v = rand_qkv(8300 + int(bf), B, T, Hq, Hkv, bf)
    qd, kd, vd = dev(q), dev(k), dev(v)
    full = host(inv().inv_attention_prefill(qd, kd, vd))
    pos = np.array([0, 15, 255, 256, 1000, 1023, 1024, 1500, 2047], np.int32)
    for p in pos:
        O = host(inv().inv_attention_decode(qd[:, p].contiguous(), kd, vd, i32(np.array([p], np.int32))))
        assert_bitwise(O[0], full[0, p], "decode pos=%d" % p)
    for s0 in (0, 1024, 2032):
        for h0 in (0, 12, 28):
            # heads h0 .. h0 + 3 share kv head h0 / 4: run them with their kv head alone
            qs = q[:, s0:s0 + 16, h0:h0 + 4].copy()
            ks, vs = k[:, h0 // 4:h0 // 4 + 1].copy(), v[:, h0 // 4:h0 // 4 + 1].copy()
            part = host(inv().inv_attention_prefill(dev(qs), dev(ks), dev(vs), q_start=s0))
            assert_bitwise(part, full[:, s0:s0 + 16, h0:h0 + 4], "rows %d, heads %d" % (s0, h0))


def test_decode_cache_length_does_not_change_rows():
    """A row's output depends only on keys 0..pos: a 140000-slot cache and one cut to pos + 1
    slots give the same bits (positions 0, 70000, 131071), and a row with an invalid
    position is NaN while the other row is unaffected."""
    import torch
    say("attn decode long cache")
    Hq, Hkv, Tbig = 4, 2, 140000
    g = torch.Generator(device="cuda")
    g.manual_seed(8300)
    K = torch.randn((2, Hkv, Tbig, D), generator=g, device="cuda")
    V = torch.randn((2, Hkv, Tbig, D), generator=g, device="cuda")
    Q = torch.randn((2, Hq, D), generator=g, device="cuda")
    for p in (0, 70000, 131071):
        pos = torch.tensor([p, -1], dtype=torch.int32, device="cuda")
        big = host(inv().inv_attention_decode(Q, K, V, pos))
        small = host(inv().inv_attention_decode(Q, K[:, :, :p + 1].contiguous(), V[:, :, :p + 1].contiguous(), pos))
        assert_bitwise(big[0], small[0], "Tmax %d vs %d at pos %d" % (Tbig, p + 1, p))
        assert np.isnan(big[1]).all() and np.isnan(small[1]).all()


def test_c2_full_prefill_equals_token_by_token_decode_and_oracle(orc):
    """8 heads x d128, 2048 tokens, bf16 Q/K/V, causal, chunk 256: prefill output equals
    2048 single-token decode calls bitwise, and the oracle at every row."""
    say("attn C2 full")
    d = synth.c2_inputs()
    q, k, v = d["q"], d["k"], d["v"]
    qd, kd, vd = bf16(q), bf16(k), bf16(v)
    pre = host(inv().inv_attention_prefill(qd, kd, vd))
    import torch
    outs = torch.empty((2048, 8, D), dtype=torch.float32, device="cuda")
    ws = torch.empty(inv().inv_attention_decode_workspace_bytes(1, 2048, 8, D), dtype=torch.uint8, device="cuda")
    posd = torch.arange(2048, dtype=torch.int32, device="cuda")
    for t in range(2048):
        inv().inv_attention_decode(qd[:, t], kd, vd, posd[t:t + 1], out=outs[t:t + 1], ws=ws)
    dec = host(outs)
    assert_bitwise(dec, pre[0], "prefill vs decode")
    say("attn C2 oracle")
    assert_bitwise(pre, orc.attention(q, k, v), "oracle")


def test_unit_values_exactly_one():
    say("attn V=1")
    q, k, _ = rand_qkv(8300, 1, 600, 2, 2)
    v = np.ones_like(k)
    O = host(inv().inv_attention_prefill(f32(q), f32(k), f32(v)))
    assert np.all(O == 1.0)


@pytest.mark.parametrize("B,T,q0,Hq,Hkv,bf", [(1, 2048, 0, 8, 8, True), (2, 900, 0, 4, 2, False),
                                              (1, 1000, 300, 8, 2, False), (3, 513, 40, 2, 1, True)])
def test_split_prefill_equals_single_task_and_oracle(orc, B, T, q0, Hq, Hkv, bf):
    """Small grids cut long row blocks into chunk tasks whose partials the merge folds: the
    same bits as the single-task kernel (and the oracle), at ragged lengths and offsets."""
    say("attn split", B, T, q0, Hq, Hkv, bf)
    m = inv()
    need = m.inv_attention_prefill_workspace_bytes(B, T, q0, Hq, D)
    assert need > 0, "shape expected to take the split path"
    q, k, v = rand_qkv(8300 + T + q0, B, q0 + T, Hq, Hkv, bf)
    qs = q[:, q0:].copy()
    split = host(m.inv_attention_prefill(dev(qs), dev(k), dev(v), q_start=q0, split=True))
    single = host(m.inv_attention_prefill(dev(qs), dev(k), dev(v), q_start=q0, split=False))
    assert_bitwise(split, single, "split vs single task")
    if B * T * Hq <= 8000:
        ref = orc.attention(q, k, v)[:, q0:]
        assert_bitwise(split, ref, "split vs oracle")


def test_split_prefill_workspace_rules():
    """Large grids need no workspace; a too-small workspace is rejected, not silently used."""
    say("attn split ws")
    m = inv()
    assert m.inv_attention_prefill_workspace_bytes(1, 16384, 0, 32, D) == 0
    assert m.inv_attention_prefill_workspace_bytes(1, 200, 0, 8, D) == 0      # one chunk per row
    need = m.inv_attention_prefill_workspace_bytes(1, 2048, 0, 8, D)
    assert need > 0
    import ctypes
    q, k, v = rand_qkv(8400, 1, 2048, 8, 8, True)
    Q, K, V = dev(q), dev(k), dev(v)
    import torch
    out = torch.empty((1, 2048, 8, D), dtype=torch.float32, device=Q.device)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=Q.device)
    from invariant_numerics_amd import binding
    rc = binding.LIB.inv_attention_prefill_ws(0, Q.data_ptr(), K.data_ptr(), V.data_ptr(), 1, 2048, 0, 2048, 8, 8, D,
                                        ctypes.c_float(0.08838834764831845), out.data_ptr(), ws.data_ptr(),
                                        need - 16, None)
    assert rc == -5
