"""Bitwise regression baseline, GPU side: the HIP library's outputs on the seeded inputs of
tests/golden/cases.py hash to the digests the oracle wrote into
tests/golden/oracle_hashes.json (one per configuration and seed)."""
import json
import os
import sys

import numpy as np
import pytest

from gpu_util import bf16, f32, host, i32, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
if GOLDEN not in sys.path:
    sys.path.insert(0, GOLDEN)

import cases as golden  # noqa: E402

STORED = json.load(open(golden.HASH_FILE))


def hip_digest(kind, d):
    import torch
    import invariant_numerics_amd as inv
    from invariant_numerics_amd.decoder import Decoder
    if kind == "lmhead":
        r = inv.inv_lmhead_logprob_top2(f32(d["h"]), bf16(d["w"]), i32(d["target"]), float(d["tau"]))
        return golden.digest(*[host(r[k]) for k in golden.LM_KEYS])
    if kind == "attention":
        return golden.digest(host(inv.inv_attention_prefill(bf16(d["q"]), bf16(d["k"]), bf16(d["v"]))))
    if kind == "gemm":
        return golden.digest(host(inv.inv_fixed_order_gemm(f32(d["x"]), bf16(d["w"]))))
    if kind == "decoder":
        toks = d["tokens"]
        B, T = toks.shape
        dec = Decoder(d["model"], device="cuda:0", batch=B, tmax=d["model"]["cos"].shape[0])
        r = dec.prefill(torch.from_numpy(toks).cuda(), block=128)
        out = {k: host(v) for k, v in r.items()}
        return golden.digest(*[np.ascontiguousarray(out[k][b]) for b in range(B) for k in golden.LM_KEYS])
    raise ValueError(kind)


@pytest.mark.parametrize("name", sorted(golden.cases()))
def test_hip_matches_stored_digest(name):
    desc, kind, build = golden.cases()[name]
    say("golden", name)
    assert hip_digest(kind, build()) == STORED[name]["sha256"], "%s (%s)" % (name, desc)
