"""Full-size decoder (4 layers, hidden 4096, 32/8 heads of 128, FFN 14336, vocab 128256,
random init, BF16 weights, FP32 compute and KV cache): bitwise equal to the oracle where the
oracle can run, and bitwise self-consistent across batch sizes, token blocks and prefill vs
token-by-token decode up to a 32k context."""
import numpy as np
import pytest

import synth
from gpu_util import assert_bitwise, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ("logprob", "margin", "top1", "top2", "recomputed")
TMAX = 32768


@pytest.fixture(scope="module")
def c5():
    say("c5 model generation")
    model = synth.decoder_model(synth.C5, TMAX)
    toks = synth.tokens(synth.SEEDS["c5_tok"], 3, TMAX, synth.C5["vocab"])
    return model, toks


@pytest.fixture(scope="module")
def dec(c5):
    from invariant_numerics_amd.decoder import Decoder
    say("c5 decoder upload")
    return Decoder(c5[0], batch=3, tmax=TMAX)


def reset(d):
    for k, v in zip(d.kc, d.vc):
        k.zero_()
        v.zero_()


def test_c5_matches_oracle_short(orc, c5, dec):
    """Every scored position of a 12-token sequence, bitwise equal to the oracle."""
    model, toks = c5
    say("c5 oracle 12 tokens")
    reset(dec)
    got = {k: host(v)[0] for k, v in dec.prefill(i32(toks[:1, :12])).items()}
    want = orc.decoder(toks[0, :12], model)
    for k in KEYS:
        assert_bitwise(got[k], want[k], k)


@pytest.mark.parametrize("act", ["bf16", "fp16"])
def test_c5_greedy_rounded_storage_matches_oracle(orc, c5, act):
    """Full-size model with BF16 / FP16 activation storage: a greedy continuation (prompt of
    8 tokens prefilled, then 3 decode steps with selective recompute) bitwise equal to the
    oracle's from-scratch loop: tokens, margins, top-2 and recompute flags."""
    from invariant_numerics_amd import agreement
    from invariant_numerics_amd.decoder import Decoder
    import torch
    model, toks = c5
    say("c5 greedy", act)
    d = Decoder(model, batch=1, tmax=64, act=act, tau=0.1)
    got = agreement.greedy(d, i32(toks[:1, :8]), 3)
    del d
    torch.cuda.empty_cache()
    want = orc.greedy(toks[0, :8], model, 3, act=act, tau=np.float32(0.1))
    for k in ("tokens", "margin", "top1", "top2", "recomputed"):
        assert_bitwise(got[k][0], want[k], "%s %s" % (act, k))


def test_c5_prefill_decode_batch_and_blocks(c5, dec):
    """T = 300 (two KV chunks): 3 sequences prefilled in token blocks of 128 equal
    (a) one sequence prefilled in one block, (b) token-by-token decode of all three."""
    import torch
    _, toks = c5
    T = 300
    td = i32(toks[:, :T])
    say("c5 prefill B=3 block 128")
    reset(dec)
    pre = {k: host(v) for k, v in dec.prefill(td, block=128).items()}
    say("c5 prefill B=1 block 4096")
    reset(dec)
    one = {k: host(v) for k, v in dec.prefill(td[2:3].contiguous(), block=4096).items()}
    for k in KEYS:
        assert_bitwise(one[k][0], pre[k][2], "batch/block %s" % k)
    say("c5 token-by-token decode")
    reset(dec)
    outs = {k: [] for k in KEYS}
    for t in range(T - 1):
        pos = torch.full((3,), t, dtype=torch.int32, device="cuda")
        r = dec.decode_step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous())
        for k in KEYS:
            outs[k].append(r[k])
    for k in KEYS:
        assert_bitwise(host(torch.stack(outs[k], dim=1)), pre[k], "prefill vs decode %s" % k)


def test_c5_32k_prefill_equals_decode_tail(c5, dec):
    """32k context: full prefill vs prefill of the first 32752 tokens followed by 15
    decode steps, at the last 15 scored positions."""
    import torch
    _, toks = c5
    td = i32(toks[:1])
    say("c5 32k full prefill")
    reset(dec)
    full = {k: host(v)[0] for k, v in dec.prefill(td, block=4096).items()}
    assert 0.1 < full["recomputed"].mean() < 0.6
    p0 = TMAX - 16
    say("c5 32k prefill", p0 + 1, "then decode")
    reset(dec)
    dec.prefill(td[:, :p0 + 1].contiguous(), block=4096)
    for t in range(p0, TMAX - 1):
        pos = torch.full((1,), t, dtype=torch.int32, device="cuda")
        r = dec.decode_step(td[:, t].contiguous(), pos, td[:, t + 1].contiguous())
        for k in KEYS:
            assert_bitwise(host(r[k]), full[k][t:t + 1], "position %d %s" % (t, k))


def test_c5_decode_batch_sizes_to_64(c5):
    """Decode at a 32k context for batch 64 (rows at different positions, synthetic seeded
    KV caches) against batch 1, 2, 4, 8, 16 and 32 on the leading rows, and row 63 moved to
    the front of a batch of one: every output bitwise equal."""
    import torch
    from invariant_numerics_amd.decoder import Decoder
    model, toks = c5
    say("c5 decode batch 64: caches")
    B = 64
    d = Decoder(model, batch=B, tmax=TMAX)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    for k in d.kc + d.vc:
        k.normal_(generator=g)
    tok = i32((toks[:, TMAX - 1][np.arange(B) % 3] + np.arange(B, dtype=np.int32)) % synth.C5["vocab"])
    tgt = i32(toks[:, TMAX - 2][np.arange(B) % 3])
    pos = torch.tensor([TMAX - 1 - 37 * b for b in range(B)], dtype=torch.int32, device="cuda")
    say("c5 decode batch 64: step")
    full = {k: host(v) for k, v in d.decode_step(tok, pos, tgt).items()}
    for b in (1, 2, 4, 8, 16, 32):
        say("c5 decode batch", b)
        r = d.decode_step(tok[:b].contiguous(), pos[:b].contiguous(), tgt[:b].contiguous())
        for k in KEYS:
            assert_bitwise(host(r[k]), full[k][:b], "batch %d %s" % (b, k))
    say("c5 decode row 63 at the front")
    for kc, vc in zip(d.kc, d.vc):
        kc[0].copy_(kc[63])
        vc[0].copy_(vc[63])
    r = d.decode_step(tok[63:64].contiguous(), pos[63:64].contiguous(), tgt[63:64].contiguous())
    for k in KEYS:
        assert_bitwise(host(r[k]), full[k][63:64], "row 63 alone %s" % k)
    del d
    torch.cuda.empty_cache()
