"""The decoder assembled from ABI calls: rmsnorm/elementwise parity, whole-model parity
with the oracle, prefill == token-by-token decode, batch and token-block invariance."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ("logprob", "margin", "top1", "top2", "recomputed")


def inv():
    import invariant_numerics_amd as m
    return m


def test_rmsnorm_matches_oracle(orc):
    say("rmsnorm")
    for M, H in ((1, 8), (7, 264), (33, 4096), (5, 14336)):
        X = synth.normal(9300 + H, (M, H))
        g = synth.to_bf16_bits(np.float32(1.0) + synth.normal(9301, (H,), 0.02))
        assert_bitwise(host(inv().inv_rmsnorm(f32(X), bf16(g))), orc.rmsnorm(X, g), "rmsnorm %d" % H)
    X = np.full((2, 4096), 0.75, np.float32)
    g = np.full(4096, 0x3F80, np.uint16)
    assert_bitwise(host(inv().inv_rmsnorm(f32(X), bf16(g))), orc.rmsnorm(X, g), "constant row")


def test_swiglu_rope_embed_match_oracle(orc):
    say("elementwise")
    G = synth.normal(9400, (9, 1000)) * np.float32(6)
    U = synth.normal(9401, (9, 1000))
    assert_bitwise(host(inv().inv_swiglu(f32(G), f32(U))), orc.swiglu(G, U), "swiglu")
    import torch
    M, Hq, Hkv, D, Tmax = 6, 4, 2, 128, 40
    QKV = synth.normal(9402, (M, (Hq + 2 * Hkv) * D))
    cos_t, sin_t = synth.rope_tables(Tmax, D)
    seq = np.array([0, 0, 1, 1, 1, 0], np.int32)
    pos = np.array([0, 5, 3, 39, 7, 20], np.int32)
    Qo = torch.empty((M, Hq, D), dtype=torch.float32, device="cuda")
    Kc = torch.zeros((2, Hkv, Tmax, D), dtype=torch.float32, device="cuda")
    Vc = torch.zeros_like(Kc)
    inv().inv_rope_kv_append(f32(QKV), Hq, Hkv, D, i32(seq), i32(pos), f32(cos_t), f32(sin_t), Qo, Kc, Vc)
    q3 = QKV[:, :Hq * D].reshape(M, Hq, D)
    k3 = QKV[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D)
    assert_bitwise(host(Qo), orc.rope(q3, pos, cos_t, sin_t), "rope q")
    kr = orc.rope(k3, pos, cos_t, sin_t)
    Kh, Vh = host(Kc), host(Vc)
    for m in range(M):
        assert_bitwise(Kh[seq[m], :, pos[m]], kr[m], "rope k row %d" % m)
        assert_bitwise(Vh[seq[m], :, pos[m]], QKV[m, (Hq + Hkv) * D:].reshape(Hkv, D), "v row %d" % m)
    table = synth.bf16_normal(9403, (50, 64))
    ids = np.array([3, 49, 0, 3], np.int32)
    assert_bitwise(host(inv().inv_embed(i32(ids), bf16(table))), orc.bf16_up(table[ids]), "embed")


@pytest.fixture(scope="module")
def small():
    return synth.decoder_model(synth.SMALL, 640, seed_base=9500, gamma_std=0.02)


def test_small_decoder_prefill_matches_oracle(orc, small):
    """2 layers, hidden 256, 4/2 heads of 128, T = 600 (three KV chunks): every scored
    position bitwise equal to the oracle, for two sequences in one batch."""
    from invariant_numerics_amd.decoder import Decoder
    say("small decoder prefill")
    toks = synth.tokens(9600, 2, 600, synth.SMALL["vocab"])
    dec = Decoder(small, batch=2, tmax=640)
    got = {k: host(v) for k, v in dec.prefill(i32(toks), block=256).items()}
    for b in range(2):
        say("small decoder oracle seq", b)
        want = orc.decoder(toks[b], small)
        for k in KEYS:
            assert_bitwise(got[k][b], want[k], "seq %d %s" % (b, k))


def test_small_decoder_prefill_equals_decode_and_batch(orc, small):
    from invariant_numerics_amd.decoder import Decoder
    import torch
    say("small decoder decode")
    T = 300
    toks = synth.tokens(9700, 3, T, synth.SMALL["vocab"])
    td = i32(toks)
    pre = {k: host(v) for k, v in Decoder(small, batch=3, tmax=320).prefill(td, block=64).items()}
    one = {k: host(v) for k, v in Decoder(small, batch=1, tmax=320).prefill(td[1:2].contiguous(),
                                                                            block=2048).items()}
    for k in KEYS:
        assert_bitwise(one[k][0], pre[k][1], "batch 1 vs 3, block 2048 vs 64: %s" % k)
    dec = Decoder(small, batch=3, tmax=320)
    outs = {k: [] for k in KEYS}
    for t in range(T - 1):
        pos = torch.full((3,), t, dtype=torch.int32, device="cuda")
        r = dec.decode_step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous())
        for k in KEYS:
            outs[k].append(host(r[k]))
    for k in KEYS:
        assert_bitwise(np.stack(outs[k], axis=1), pre[k], "prefill vs decode %s" % k)


def test_small_decoder_graph_replays_equal_eager(small):
    """One decode step captured in a graph and replayed at every position, with eager work
    and synchronisations between replays: every replay bitwise equal to eager decode."""
    from invariant_numerics_amd.decoder import Decoder
    import torch
    say("small decoder graph decode")
    T = 280
    toks = synth.tokens(9800, 2, T, synth.SMALL["vocab"])
    td = i32(toks)
    eager = Decoder(small, batch=2, tmax=320)
    ref = []
    for t in range(T - 1):
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        r = eager.decode_step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous())
        ref.append({k: host(v) for k, v in r.items()})
    gdec = Decoder(small, batch=2, tmax=320)
    # capture after a prefill of the first 100 tokens: capturing must not disturb the cache
    gdec.prefill(td[:, :101].contiguous(), block=64)
    step = gdec.decode_graph()
    for t in range(100, T - 1):
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        r = step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous())
        got = {k: host(v) for k, v in r.items()}
        _ = torch.randn(1000, device="cuda").sum().item()   # eager work between replays
        for k in KEYS:
            assert_bitwise(got[k], ref[t][k], "graph replay %d %s" % (t, k))


def test_small_decoder_multi_step_graph_equals_eager(small):
    """K consecutive decode steps captured as one graph and replayed (K = 5, windows of
    positions across a 256-key chunk boundary, eager work between replays): every step of
    every replay bitwise equal to eager decode at that position, and the KV cache the same."""
    from invariant_numerics_amd.decoder import Decoder
    import torch
    say("small decoder multi-step graph")
    T, K = 280, 5
    toks = synth.tokens(9810, 2, T, synth.SMALL["vocab"])
    td = i32(toks)
    eager = Decoder(small, batch=2, tmax=320)
    ref = []
    for t in range(T - 1):
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        r = eager.decode_step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous())
        ref.append({k: host(v) for k, v in r.items()})
    gdec = Decoder(small, batch=2, tmax=320)
    gdec.prefill(td[:, :241].contiguous(), block=64)
    run = gdec.decode_graph_steps(K)
    for t0 in range(240, T - K, K):
        tok = torch.stack([td[:, t] for t in range(t0, t0 + K)]).contiguous()
        pos = torch.stack([torch.full((2,), t, dtype=torch.int32, device="cuda") for t in range(t0, t0 + K)])
        tgt = torch.stack([td[:, t + 1] for t in range(t0, t0 + K)]).contiguous()
        outs = run(tok, pos, tgt)
        got = [{k: host(v) for k, v in o.items()} for o in outs]
        _ = torch.randn(1000, device="cuda").sum().item()   # eager work between replays
        for i in range(K):
            for k in KEYS:
                assert_bitwise(got[i][k], ref[t0 + i][k], "multi-step graph %d %s" % (t0 + i, k))
    last = t0 + K
    for li in range(len(eager.kc)):
        assert_bitwise(host(gdec.kc[li][:, :, :last]), host(eager.kc[li][:, :, :last]), "k cache %d" % li)
        assert_bitwise(host(gdec.vc[li][:, :, :last]), host(eager.vc[li][:, :, :last]), "v cache %d" % li)
