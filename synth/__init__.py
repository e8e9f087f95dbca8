"""Seeded synthetic inputs shared by the HIP path's tests/bench and by the oracle.

This module holds input generation only: random draws, integer ids and the RoPE
angle tables that a model carries as constants.  It contains none of the method's
arithmetic; BF16 storage of drawn weights uses PyTorch's own float->bfloat16
conversion.  Host arrays produced here are handed unchanged to both sides.

Recipe (stated once, used everywhere):
  * bit generator: NumPy Philox, one stream per tensor, key = ``seed``; tensors larger
    than one chunk are filled chunk by chunk, chunk ``i`` drawn from the stream jumped
    ``i`` times, so the values do not depend on the number of threads used;
  * normals drawn in float32 (``standard_normal``) then multiplied by the std in
    float32; BF16 tensors are those float32 draws rounded to nearest-even by PyTorch;
  * seeds: 1000 * config + tensor id (configs 1..5), see ``SEEDS``.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CHUNK = 1 << 24  # elements per independently seeded chunk

SEEDS = {
    # C1: LM-head logprob only
    "c1_h": 1001, "c1_w": 1002, "c1_tgt": 1003,
    # C2: attention consistency
    "c2_q": 2001, "c2_k": 2002, "c2_v": 2003,
    # C3: batch-invariant GEMM
    "c3_x": 3001, "c3_w4096": 3002, "c3_w14336": 3003, "c3_wdown": 3004, "c3_xdown": 3005,
    # C4: 7B-shape LM head
    "c4_h": 4001, "c4_w": 4002, "c4_tgt": 4003, "c4_stress": 4004,
    # C5: Llama-shaped decoder
    "c5_emb": 5001, "c5_head": 5002, "c5_tok": 5003, "c5_layer": 5100,
}


def _gen(seed, i=0):
    bg = np.random.Philox(seed)
    if i:
        bg = bg.jumped(i)
    return np.random.Generator(bg)


def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def normal(seed, shape, std=1.0):
    """float32 N(0, std^2) draws, chunked and seeded as described above."""
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(i):
        lo, hi = i * CHUNK, min(n, (i + 1) * CHUNK)
        g = _gen(seed, i)
        g.standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks <= 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def to_bf16_bits(a):
    """float32 array -> BF16 bit patterns (uint16), rounded by PyTorch's conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_normal(seed, shape, std=0.02):
    return to_bf16_bits(normal(seed, shape, std))


def uniform_int(seed, shape, high):
    return _gen(seed).integers(0, high, size=shape, dtype=np.int64).astype(np.int32)


def permutation(seed, n):
    return _gen(seed).permutation(n)


def rope_tables(tmax, d, theta=500000.0):
    """Rotate-half RoPE tables, cos/sin of t * theta^(-2i/d) for t < tmax, i < d/2,
    evaluated in float64 and stored as float32 (a model constant, like a weight)."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = theta ** (-2.0 * i / d)
    ang = np.arange(tmax, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


# ------------------------------------------------------------------ configs --

def c1_inputs(rows=64, hidden=256, vocab=4096):
    """LM-head-only config: h fp32 N(0,1), W bf16 N(0, 0.02), uniform targets."""
    return dict(h=normal(SEEDS["c1_h"], (rows, hidden)),
                w=bf16_normal(SEEDS["c1_w"], (vocab, hidden), 0.02),
                target=uniform_int(SEEDS["c1_tgt"], (rows,), vocab))


def c2_inputs(heads=8, seq=2048, d=128):
    """Attention config: bf16 Q/K/V N(0,1), laid out [1, T, H, D] (Q) and [1, H, T, D] (K, V)."""
    q = bf16_normal(SEEDS["c2_q"], (heads, seq, d), 1.0)
    k = bf16_normal(SEEDS["c2_k"], (heads, seq, d), 1.0)
    v = bf16_normal(SEEDS["c2_v"], (heads, seq, d), 1.0)
    return dict(q=np.ascontiguousarray(q.transpose(1, 0, 2))[None], k=k[None], v=v[None])


def c3_inputs(n=4096, k=4096, rows=512, seed_w=None, seed_x=None):
    """GEMM config: X fp32 N(0,1) [rows, k], W bf16 N(0, 0.02) [n, k]."""
    sw = seed_w if seed_w is not None else (SEEDS["c3_w4096"] if n == 4096 else SEEDS["c3_w14336"])
    sx = seed_x if seed_x is not None else SEEDS["c3_x"]
    return dict(x=normal(sx, (rows, k)), w=bf16_normal(sw, (n, k), 0.02))


def c4_inputs(rows=256, hidden=4096, vocab=128256, stress=False):
    """7B-shape LM head: h fp32 N(0,1) [rows, hidden], W bf16 N(0, 0.02) [vocab, hidden].
    stress=True makes near-tied logits: W row 2i+1 = W row 2i + N(0, 1e-3) (before BF16)."""
    w = normal(SEEDS["c4_w"], (vocab, hidden), 0.02)
    if stress:
        d = normal(SEEDS["c4_stress"], (vocab // 2, hidden), 1e-3)
        w[1::2][: vocab // 2] = w[0::2][: vocab // 2] + d
    return dict(h=normal(SEEDS["c4_h"], (rows, hidden)), w=to_bf16_bits(w),
                target=uniform_int(SEEDS["c4_tgt"], (rows,), vocab))


C5 = dict(hidden=4096, hq=32, hkv=8, d=128, ffn=14336, vocab=128256, layers=4, theta=500000.0)
TINY = dict(hidden=64, hq=4, hkv=2, d=16, ffn=160, vocab=512, layers=2, theta=10000.0)
# smallest shape the GPU path accepts (head dim 128), for fast whole-decoder parity runs
SMALL = dict(hidden=256, hq=4, hkv=2, d=128, ffn=512, vocab=1000, layers=2, theta=500000.0)


def decoder_model(cfg, tmax, seed_base=None, gamma_std=0.0):
    """Random-init Llama-shaped decoder (all linears and the embedding N(0, 0.02) in BF16,
    untied head; RMSNorm gains 1.0, or bf(1 + N(0, gamma_std)) when gamma_std > 0)."""
    H, Hq, Hkv, D, F, V, L = (cfg[k] for k in ("hidden", "hq", "hkv", "d", "ffn", "vocab", "layers"))
    base = SEEDS["c5_layer"] if seed_base is None else seed_base
    one = np.full(H, 0x3F80, np.uint16)

    def gamma(s):
        if gamma_std <= 0:
            return one.copy()
        return to_bf16_bits(np.float32(1.0) + normal(s, (H,), gamma_std))

    layers = []
    for li in range(L):
        s = base + 10 * li
        layers.append(dict(
            g1=gamma(s + 0),
            wqkv=bf16_normal(s + 1, ((Hq + 2 * Hkv) * D, H)),
            wo=bf16_normal(s + 2, (H, Hq * D)),
            g2=gamma(s + 3),
            w13=bf16_normal(s + 4, (2 * F, H)),
            w2=bf16_normal(s + 5, (H, F)),
        ))
    cos_t, sin_t = rope_tables(tmax, D, cfg["theta"])
    emb_seed = SEEDS["c5_emb"] if seed_base is None else seed_base + 1
    head_seed = SEEDS["c5_head"] if seed_base is None else seed_base + 2
    return dict(cfg=dict(cfg), emb=bf16_normal(emb_seed, (V, H)), layers=layers,
                gf=gamma(base + 9), whead=bf16_normal(head_seed, (V, H)), cos=cos_t, sin=sin_t)


def tokens(seed, batch, seq, vocab):
    return uniform_int(seed, (batch, seq), vocab)
