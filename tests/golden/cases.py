"""Seeded inputs of the bitwise regression baseline (tests/golden/oracle_hashes.json) and the
digest both sides take of their outputs.  Input recipes only: no arithmetic of the method."""
import hashlib
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HASH_FILE = os.path.join(HERE, "oracle_hashes.json")
LM_KEYS = ("logprob", "margin", "top1", "top2", "recomputed")


def digest(*arrays):
    """SHA-256 over the arrays' little-endian bytes in order (float32, int32, uint8)."""
    h = hashlib.sha256()
    for a in arrays:
        a = np.ascontiguousarray(a)
        assert a.dtype in (np.float32, np.int32, np.uint8), a.dtype
        h.update(a.astype(a.dtype.newbyteorder("<"), copy=False).tobytes())
    return h.hexdigest()


def cases():
    """Name -> (description, input builder).  Each builder returns a dict of host arrays; the
    same builders feed the oracle here and the HIP path in the GPU test."""
    def c1():
        return dict(synth.c1_inputs(), tau=np.float32(0.1))

    def c2():
        return synth.c2_inputs()

    def c3(n, k, seed_w, seed_x):
        def f():
            return dict(x=synth.normal(seed_x, (512, k))[:16], w=synth.bf16_normal(seed_w, (n, k)))
        return f

    def c4(stress):
        def f():
            d = synth.c4_inputs(rows=8, stress=stress)
            return dict(h=d["h"], w=d["w"], target=d["target"], tau=np.float32(0.1))
        return f

    def c5_small():
        m = synth.decoder_model(synth.SMALL, 320, seed_base=9900, gamma_std=0.02)
        return dict(model=m, tokens=synth.tokens(9901, 2, 300, synth.SMALL["vocab"]))

    def c5_full():
        m = synth.decoder_model(synth.C5, 64)
        return dict(model=m, tokens=synth.tokens(synth.SEEDS["c5_tok"], 1, 12, synth.C5["vocab"]))

    S = synth.SEEDS
    return {
        "c1_lmhead_v4096_k256_64rows": ("LM head, 64 rows, tau 0.1", "lmhead", c1),
        "c2_attention_8x2048_bf16": ("attention prefill, 8 heads x 2048, BF16 Q/K/V", "attention", c2),
        "c3_gemm_4096x4096_16rows": ("GEMM, rows 0..15 of X, W 4096 x 4096", "gemm",
                                     c3(4096, 4096, S["c3_w4096"], S["c3_x"])),
        "c3_gemm_14336x4096_16rows": ("GEMM, rows 0..15 of X, W 14336 x 4096", "gemm",
                                      c3(14336, 4096, S["c3_w14336"], S["c3_x"])),
        "c3_gemm_4096x14336_16rows": ("GEMM, rows 0..15 of X, W 4096 x 14336 (down projection)", "gemm",
                                      c3(4096, 14336, S["c3_wdown"], S["c3_xdown"])),
        "c4_lmhead_v128256_8rows": ("LM head, vocab 128256, rows 0..7, tau 0.1", "lmhead", c4(False)),
        "c4_lmhead_v128256_8rows_stress": ("LM head, near-tied weight rows, rows 0..7, tau 0.1", "lmhead",
                                           c4(True)),
        "c5_small_decoder_2x300": ("2-layer decoder (hidden 256, head dim 128), 2 x 300 tokens", "decoder",
                                   c5_small),
        "c5_decoder_12_tokens": ("4-layer Llama-8B-shaped decoder, first 12 tokens of sequence 0", "decoder",
                                 c5_full),
    }


