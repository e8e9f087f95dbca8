"""Low-precision activation storage and greedy generation on the GPU against the oracle:
the rounding entry point (BF16 / FP16 / copy, strided, in place), RoPE + cache append with
rounded outputs, the BF16- and FP16-storage decoders (prefill == oracle, prefill == decode),
and greedy continuations under several policies (tokens, margins, top-2 and recompute
flags bitwise equal to the oracle's from-scratch greedy loop; batch composition changes
nothing)."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ("logprob", "margin", "top1", "top2", "recomputed")
GKEYS = ("tokens", "margin", "top1", "top2", "recomputed")


def inv():
    import invariant_numerics_amd as m
    return m


def patterns(n, seed):
    """Random bit patterns (every class: NaN, inf, subnormal, huge) plus the FP16 and BF16
    rounding edges: ties around 1, the subnormal range, the overflow threshold."""
    rng = np.random.default_rng(seed)
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    edges = [np.arange(0x3F800000, 0x3F800000 + 0x4000, dtype=np.uint32),       # 1 .. 1 + 2^-9
             np.arange(0x33000000 - 64, 0x33000000 + 64, dtype=np.uint32),      # ~2^-25
             np.arange(0x387FE000, 0x38802000, dtype=np.uint32),                # ~2^-14
             np.arange(0x477FE000, 0x47801000, dtype=np.uint32),                # ~65504 .. 2^16
             np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0xFFBFFFFF, 0x7F7FFFFF,
                       0x00000001, 0x807FFFFF], np.uint32)]
    edges = np.concatenate(edges)
    return np.concatenate([u, edges, edges | 0x80000000]).view(np.float32)


@pytest.mark.parametrize("fmt", ["bf16", "fp16", "fp32"])
def test_round_activations_matches_oracle(orc, fmt):
    import torch
    x = patterns(1 << 20, 31)
    n = x.size - x.size % 28
    X = x[:n].reshape(-1, 28)
    say("round activations", fmt, X.shape)
    want = orc.round_act(X, fmt)
    dX = f32(X)
    assert_bitwise(host(inv().inv_round_activations(dX, fmt)), want, fmt + " vector path")
    # strided view with odd width (scalar path), written into a strided output
    sub = dX[:, 1:26]
    out = torch.full((X.shape[0], 30), 7.0, device="cuda")
    inv().inv_round_activations(sub, fmt, out=out[:, 2:27])
    o = host(out)
    assert_bitwise(o[:, 2:27], want[:, 1:26], fmt + " strided")
    assert np.all(o[:, :2] == 7.0) and np.all(o[:, 27:] == 7.0)
    # in place
    inv().inv_round_activations(dX, fmt, out=dX)
    assert_bitwise(host(dX), want, fmt + " in place")


def test_round_activations_rejects_bad_arguments():
    import torch
    L = inv().binding.LIB
    x = torch.zeros((4, 8), device="cuda")
    p = x.data_ptr()
    s = torch.cuda.current_stream().cuda_stream
    assert L.inv_round_activations(p, 4, 8, 8, 3, p, 8, s) == -4          # unknown format
    assert L.inv_round_activations(p, 4, 8, 7, 0, p, 8, s) == -2          # stride < width
    assert L.inv_round_activations(p + 2, 4, 8, 8, 0, p, 8, s) == -3      # misaligned
    assert L.inv_round_activations(None, 4, 8, 8, 0, p, 8, s) == -1
    assert L.inv_round_activations(p, 0, 8, 8, 0, p, 8, s) == 0           # empty: nothing to do


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_rope_kv_append_rounded_outputs(orc, fmt):
    import torch
    say("rope rounded", fmt)
    M, Hq, Hkv, D, Tmax = 6, 4, 2, 128, 40
    QKV = orc.round_act(synth.normal(9402, (M, (Hq + 2 * Hkv) * D)) * np.float32(3), fmt)
    cos_t, sin_t = synth.rope_tables(Tmax, D)
    seq = np.array([0, 0, 1, 1, 1, 0], np.int32)
    pos = np.array([0, 5, 3, 39, 7, 20], np.int32)
    Qo = torch.empty((M, Hq, D), dtype=torch.float32, device="cuda")
    Kc = torch.zeros((2, Hkv, Tmax, D), dtype=torch.float32, device="cuda")
    Vc = torch.zeros_like(Kc)
    inv().inv_rope_kv_append(f32(QKV), Hq, Hkv, D, i32(seq), i32(pos), f32(cos_t), f32(sin_t), Qo, Kc, Vc,
                             fmt=fmt)
    q3 = QKV[:, :Hq * D].reshape(M, Hq, D)
    k3 = QKV[:, Hq * D:(Hq + Hkv) * D].reshape(M, Hkv, D)
    assert_bitwise(host(Qo), orc.round_act(orc.rope(q3, pos, cos_t, sin_t), fmt), "rope q")
    kr = orc.round_act(orc.rope(k3, pos, cos_t, sin_t), fmt)
    Kh, Vh = host(Kc), host(Vc)
    for m in range(M):
        assert_bitwise(Kh[seq[m], :, pos[m]], kr[m], "rope k row %d" % m)
        assert_bitwise(Vh[seq[m], :, pos[m]], QKV[m, (Hq + Hkv) * D:].reshape(Hkv, D), "v row %d" % m)


@pytest.fixture(scope="module")
def small():
    return synth.decoder_model(synth.SMALL, 640, seed_base=9500, gamma_std=0.02)


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_rounded_decoder_prefill_matches_oracle(orc, small, act):
    """2 layers, hidden 256, T = 300 (two KV chunks), two sequences, token blocks of 128."""
    from invariant_numerics_amd.decoder import Decoder
    say("rounded decoder prefill", act)
    toks = synth.tokens(9610, 2, 300, synth.SMALL["vocab"])
    dec = Decoder(small, batch=2, tmax=320, act=act)
    got = {k: host(v) for k, v in dec.prefill(i32(toks), block=128).items()}
    for b in range(2):
        want = orc.decoder(toks[b], small, act=act)
        for k in KEYS:
            assert_bitwise(got[k][b], want[k], "%s seq %d %s" % (act, b, k))


def test_rounded_decoder_prefill_equals_decode_and_graph(small):
    """FP16 storage: token-by-token decode (eager and graph-replayed) equals prefill."""
    from invariant_numerics_amd.decoder import Decoder
    import torch
    say("rounded decoder decode fp16")
    T = 160
    toks = synth.tokens(9710, 2, T, synth.SMALL["vocab"])
    td = i32(toks)
    pre = {k: host(v) for k, v in Decoder(small, batch=2, tmax=192, act="fp16").prefill(td, block=64).items()}
    dec = Decoder(small, batch=2, tmax=192, act="fp16")
    gdec = Decoder(small, batch=2, tmax=192, act="fp16")
    gdec.prefill(td[:, :41].contiguous(), block=64)
    step = gdec.decode_graph()
    for t in range(T - 1):
        pos = torch.full((2,), t, dtype=torch.int32, device="cuda")
        r = {k: host(v) for k, v in dec.decode_step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous()).items()}
        for k in KEYS:
            assert_bitwise(r[k], pre[k][:, t], "decode %d %s" % (t, k))
        if t >= 40:
            g = {k: host(v) for k, v in step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous()).items()}
            for k in KEYS:
                assert_bitwise(g[k], pre[k][:, t], "graph %d %s" % (t, k))


@pytest.mark.parametrize("act,tau", [("fp32", 0.1), ("bf16", 0.0), ("fp16", 0.1), ("fp16", np.inf)])
def test_greedy_matches_oracle(orc, small, act, tau):
    """Greedy continuation (prefill of the prompt, then decode steps feeding back top-1)
    against the oracle's loop that rescores the whole sequence from scratch at every step."""
    from invariant_numerics_amd import agreement
    from invariant_numerics_amd.decoder import Decoder
    say("greedy", act, tau)
    P, S = 12, 10
    prompts = synth.tokens(9810, 2, P, synth.SMALL["vocab"])
    dec = Decoder(small, batch=2, tmax=64, act=act, tau=tau)
    got = agreement.greedy(dec, i32(prompts), S)
    for b in range(2):
        want = orc.greedy(prompts[b], small, S, act=act, tau=np.float32(tau))
        for k in GKEYS:
            assert_bitwise(got[k][b], want[k], "%s tau %s prompt %d %s" % (act, tau, b, k))


def test_greedy_batch_invariant(small):
    """The same prompt continued alone and inside a batch of three: identical records."""
    from invariant_numerics_amd import agreement
    from invariant_numerics_amd.decoder import Decoder
    say("greedy batch invariance")
    prompts = synth.tokens(9820, 3, 20, synth.SMALL["vocab"])
    three = agreement.greedy(Decoder(small, batch=3, tmax=64, act="bf16"), i32(prompts), 24)
    one = agreement.greedy(Decoder(small, batch=1, tmax=64, act="bf16"), i32(prompts[1:2]), 24)
    for k in GKEYS:
        assert_bitwise(one[k][0], three[k][1], "batch 1 vs 3 " + k)
