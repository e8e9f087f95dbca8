"""Throughput of the four smaller configurations on one GPU, and decode of the C5 decoder at
batch 1 to 64 (its prefill scoring is bench.py).

Seeded synthetic inputs from ``synth`` (the same arrays the parity tests use); every timing
is the median of HIP-event-bracketed repetitions on the current stream, inputs resident in
HBM.  Prints one JSON object per measurement:
  * C1: LM head, hidden 256, vocab 4096, 64 tokens as 64 / B calls of batch B;
  * C2: causal attention, 8 heads x 2048 x 128, BF16 inputs: the whole prefill, and decode
    calls at every 8th position;
  * C3: fixed-order GEMM at M in {1, 3, 16, 64, 257, 512} for the 4096 x 4096, 14336 x 4096
    and 4096 x 14336 weights, rotating over weight copies larger than the 256 MB last-level
    cache so every call reads its weights from HBM;
  * C4: LM head, hidden 4096, vocab 128256, B = 1 .. 256 (bytes count a second weight read
    when any row is recomputed and B > 16; up to 16 rows the FP32 logits share the sweep);
  * C5 decode: graph-replayed decode steps of the 4-layer decoder at a 32k context for
    B = 1, 4, 16, 64 (seeded random KV caches; bytes = weights + the KV read once).
Usage: python bench_configs.py
"""
import json, os, sys
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import numpy as np, torch
import synth
import invariant_numerics_amd as inv
dev = torch.device("cuda:0")
def timeit(fn, reps=10, warm=2):
    for _ in range(warm): fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        a.record(); fn(); b.record(); torch.cuda.synchronize(); ts.append(a.elapsed_time(b) * 1e-3)
    return float(np.median(ts))
def out(**k): print(json.dumps(k), flush=True)
def bf(a): return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
def f32(a): return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
HBM = 8000.0
# ---- C1: LM head hidden 256, vocab 4096, 64 tokens at B = 1, 2, 4, 8
d = synth.c1_inputs()
H, W, T = f32(d["h"]), bf(d["w"]), torch.from_numpy(np.ascontiguousarray(d["target"], np.int32)).to(dev)
for B in (1, 2, 4, 8):
    def run():
        for s in range(0, 64, B):
            inv.inv_lmhead_logprob_top2(H[s:s + B], W, T[s:s + B], 0.1)
    t = timeit(run)
    out(config="C1", batch=B, calls=64 // B, us_per_call=round(t / (64 // B) * 1e6, 1), tokens_per_s=round(64 / t, 1))
# ---- C2: attention 8 heads x 2048 x d128, bf16, causal
d = synth.c2_inputs()
q, k, v = bf(d["q"]), bf(d["k"]), bf(d["v"])
t = timeit(lambda: inv.inv_attention_prefill(q, k, v))
pairs = 8 * 2048 * 2049 // 2
out(config="C2", op="prefill", ms=round(t * 1e3, 3), tflops=round(pairs * 512 / t / 1e12, 2), frac_fp32_peak=round(pairs * 512 / t / 157.3e12, 3))
ws = torch.empty(inv.inv_attention_decode_workspace_bytes(1, 2048, 8, 128), dtype=torch.uint8, device=dev)
o1 = torch.empty((1, 8, 128), dtype=torch.float32, device=dev)
posd = torch.arange(2048, dtype=torch.int32, device=dev)
def dec():
    for tt in range(0, 2048, 8):
        inv.inv_attention_decode(q[:, tt], k, v, posd[tt:tt + 1], out=o1, ws=ws)
t = timeit(dec, reps=3, warm=1)
out(config="C2", op="decode", us_per_call=round(t / 256 * 1e6, 2), note="256 calls at positions 0, 8, ..., 2040")
# ---- C3: GEMM, weights cold (rotating copies > the 256 MB last-level cache)
for (n, kk) in ((4096, 4096), (14336, 4096), (4096, 14336)):
    dd = synth.c3_inputs(n=n, k=kk, rows=512, seed_w=synth.SEEDS["c3_wdown"] if kk == 14336 else None,
                         seed_x=synth.SEEDS["c3_xdown"] if kk == 14336 else None)
    X = f32(dd["x"]); W0 = bf(dd["w"])
    ncp = max(2, int(600e6 // (n * kk * 2)) + 1)
    Ws = [W0] + [W0.clone() for _ in range(ncp - 1)]
    for M in (1, 3, 16, 64, 257, 512):
        Y = torch.empty((M, n), dtype=torch.float32, device=dev)
        ctr = [0]
        def g():
            inv.inv_fixed_order_gemm(X[:M], Ws[ctr[0] % len(Ws)], out=Y); ctr[0] += 1
        t = timeit(g, reps=12)
        by = n * kk * 2 + 4 * M * kk + 4 * M * n
        out(config="C3", N=n, K=kk, M=M, us=round(t * 1e6, 1), tflops=round(2 * M * n * kk / t / 1e12, 2),
            hbm_gbs=round(by / t / 1e9, 1), frac_hbm=round(by / t / 1e9 / HBM, 3), frac_fp32=round(2 * M * n * kk / t / 157.3e12, 3))
    del Ws
# ---- C4: LM head hidden 4096, vocab 128256, B = 1 .. 256
d = synth.c4_inputs()
H, W, T = f32(d["h"]), bf(d["w"]), torch.from_numpy(np.ascontiguousarray(d["target"], np.int32)).to(dev)
for B in (1, 2, 4, 8, 16, 32, 64, 128, 256):
    r = inv.inv_lmhead_logprob_top2(H[:B], W, T[:B], 0.1)
    nrec = int(r["recomputed"].sum().item())
    t = timeit(lambda: inv.inv_lmhead_logprob_top2(H[:B], W, T[:B], 0.1), reps=6)
    wb = 1050673152
    by = wb * (2 if (nrec and B > 16) else 1) + B * 4096 * 4
    out(config="C4", batch=B, recomputed=nrec, us=round(t * 1e6, 1), tokens_per_s=round(B / t, 1),
        hbm_gbs=round(by / t / 1e9, 1), frac_hbm=round(by / t / 1e9 / HBM, 3),
        tflops=round(2 * 128256 * 4096 * (B + nrec) / t / 1e12, 2))
# ---- C5: decode steps of the 4-layer decoder at a 32k context, batch 1 .. 64 (graph replay;
# KV caches filled with seeded random values, every row at its own position near 32k)
from invariant_numerics_amd.decoder import Decoder
cfg = dict(synth.C5)
T5 = 32768
model = synth.decoder_model(cfg, T5)
dec5 = Decoder(model, device=dev, batch=64, tmax=T5)
g5 = torch.Generator(device=dev); g5.manual_seed(5005)
for k in dec5.kc + dec5.vc:
    k.normal_(generator=g5)
H5, F5, V5, L5 = cfg["hidden"], cfg["ffn"], cfg["vocab"], cfg["layers"]
QKV5 = (cfg["hq"] + 2 * cfg["hkv"]) * cfg["d"]
body_w = L5 * 2 * (QKV5 * H5 + H5 * cfg["hq"] * cfg["d"] + 2 * F5 * H5 + H5 * F5)
head_w = 2 * V5 * H5
for B in (1, 4, 16, 64):
    step = dec5.decode_graph(B)
    tok = torch.randint(0, V5, (B,), dtype=torch.int32, device=dev, generator=g5)
    tgt = torch.randint(0, V5, (B,), dtype=torch.int32, device=dev, generator=g5)
    pos = torch.tensor([T5 - 17 - 5 * b for b in range(B)], dtype=torch.int32, device=dev)
    r = step(tok, pos, tgt)
    nrec = int(r["recomputed"].sum().item())
    t = timeit(lambda: step(tok, pos, tgt), reps=10)
    kv = L5 * 2 * cfg["hkv"] * cfg["d"] * 4 * int((pos + 1).sum().item())
    by = body_w + head_w * (2 if (nrec and B > 16) else 1) + kv
    out(config="C5", op="decode", context=T5, batch=B, recomputed=nrec, ms_per_step=round(t * 1e3, 3),
        tokens_per_s=round(B / t, 1), hbm_gbs=round(by / t / 1e9, 1), frac_hbm=round(by / t / 1e9 / HBM, 3))
print("done", flush=True)
