"""Throughput of the four smaller configurations on one GPU, and decode of the C5 decoder at
batch 1 to 64 (its prefill scoring is bench.py).

Seeded synthetic inputs from ``synth`` (the same arrays the parity tests use); every timing
is the median of HIP-event-bracketed repetitions on the current stream, inputs resident in
HBM.  Prints one JSON object per measurement, and per configuration the bitwise match rates of
GPU outputs across batch sizes (C1, C3, C4) and between prefill and decode (C2):
  * C1: LM head, hidden 256, vocab 4096, 64 tokens as 64 / B calls of batch B, issued call by
    call from Python and, captured once as a HIP graph, replayed;
  * C2: causal attention, 8 heads x 2048 x 128, BF16 inputs: the whole prefill (four calls
    back to back per timing, buffers allocated beforehand), and decode calls at every 8th
    position;
  * C3: fixed-order GEMM at M in {1, 3, 16, 64, 257, 512} for the 4096 x 4096, 14336 x 4096
    and 4096 x 14336 weights, rotating over weight copies larger than the 256 MB last-level
    cache so every call reads its weights from HBM; eight calls back to back per timing (the
    launch gaps count, the host's time to issue a call does not);
  * C4: LM head, hidden 4096, vocab 128256, B = 1 .. 256, four calls back to back per timing
    with their buffers allocated beforehand (bytes count a second weight read when any row is
    recomputed and B > 32; up to 32 rows the FP32 logits share the sweep);
  * C5 decode: decode steps of the 4-layer decoder at a 32k context for B = 1, 4, 16, 64, four
    consecutive steps captured as one HIP graph and replayed (seeded random KV caches; bytes =
    weights + the KV read once);
  * probes: the practical ceilings the kernels are compared with -- a plain 16-byte read
    stream over 4 GiB (inv_read_stream_probe), torch's device copy, and the FP32 matrix
    instruction rates (inv_mfma_rate_probe) at 1, 2, 4 and 8 wavefronts per SIMD.
Usage: python bench_configs.py [section ...]   (sections: C1 C2 C3 C4 C5 probes; default all)
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
def match(a, b):
    """Bitwise match rate: equal 32-bit words / compared words (float32 outputs compared as bits)."""
    a, b = a.contiguous(), b.contiguous()
    if a.dtype == torch.float32:
        a, b = a.view(torch.int32), b.view(torch.int32)
    return round(float((a == b).sum().item()) / a.numel(), 6)
LMK = ("logprob", "margin", "top1", "top2", "recomputed")
def bf(a): return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
def f32(a): return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
HBM = 8000.0
SECTIONS = set(sys.argv[1:]) or {"C1", "C2", "C3", "C4", "C5", "probes"}
# ---- probes: read stream, copy, FP32 matrix instruction rates
if "probes" in SECTIONS:
    src = torch.empty(1 << 30, dtype=torch.float32, device=dev).fill_(1.0)   # 4 GiB
    nb = src.numel() * 4
    for grid in (2048, 4096, 8192, 16384):
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        t = timeit(lambda: inv.inv_read_stream_probe(src, grid=grid, sink=sink), reps=8)
        out(probe="read_stream", bytes=nb, grid=grid, us=round(t * 1e6, 1), gbs=round(nb / t / 1e9, 1),
            frac_hbm=round(nb / t / 1e9 / HBM, 3))
    dst = torch.empty_like(src[: src.numel() // 2])
    t = timeit(lambda: dst.copy_(src[: src.numel() // 2]), reps=8)
    out(probe="copy", bytes_read_plus_write=nb, us=round(t * 1e6, 1), gbs=round(nb / t / 1e9, 1))
    del src, dst
    for shape, fl in ((0, 2048), (1, 4096)):
        for wpc in (4, 8, 16, 32):
            grid = 256 * wpc // 4
            iters = 20000 if shape == 0 else 10000
            buf = torch.empty(grid * 256, dtype=torch.float32, device=dev)
            t = timeit(lambda: inv.inv_mfma_rate_probe(shape, iters, wpc, out=buf), reps=5)
            flops = grid * 4 * iters * 8 * fl
            out(probe="mfma_f32", instr=("16x16x4" if shape == 0 else "32x32x2"), waves_per_simd=wpc // 4,
                us=round(t * 1e6, 1), tflops=round(flops / t / 1e12, 2), frac_fp32_peak=round(flops / t / 157.3e12, 3))
# ---- C1: LM head hidden 256, vocab 4096, 64 tokens at B = 1, 2, 4, 8
if "C1" in SECTIONS:
    d = synth.c1_inputs()
    H, W, T = f32(d["h"]), bf(d["w"]), torch.from_numpy(np.ascontiguousarray(d["target"], np.int32)).to(dev)
    c1out = {}
    for B in (1, 2, 4, 8):
        ws1 = torch.empty(inv.inv_lmhead_workspace_bytes(B, 256, 4096), dtype=torch.uint8, device=dev)
        r1 = inv.inv_lmhead_logprob_top2(H[:B], W, T[:B], 0.1, ws=ws1)
        def run():
            for s in range(0, 64, B):
                inv.inv_lmhead_logprob_top2(H[s:s + B], W, T[s:s + B], 0.1, ws=ws1, out=r1)
        t = timeit(run)
        # the 64 rows as computed at this batch size, for the across-batch match rate
        c1rows = {k: [] for k in LMK}
        for s in range(0, 64, B):
            rr = inv.inv_lmhead_logprob_top2(H[s:s + B], W, T[s:s + B], 0.1, ws=ws1)
            for k in LMK: c1rows[k].append(rr[k].clone())
        c1out[B] = {k: torch.cat(v) for k, v in c1rows.items()}
        # the same 64 / B calls captured once as a HIP graph and replayed: the device time,
        # without the host's time to issue each call
        run()
        torch.cuda.synchronize()
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            run()
        tg = timeit(g1.replay)
        out(config="C1", batch=B, calls=64 // B, us_per_call=round(t / (64 // B) * 1e6, 1), tokens_per_s=round(64 / t, 1),
            graph_us_per_call=round(tg / (64 // B) * 1e6, 1), graph_tokens_per_s=round(64 / tg, 1))
    out(config="C1", bitwise_across_batch_vs_b1={B: min(match(c1out[B][k], c1out[1][k]) for k in LMK) for B in c1out},
        words_per_batch=64 * len(LMK))
# ---- C2: attention 8 heads x 2048 x d128, bf16, causal
if "C2" in SECTIONS:
    d = synth.c2_inputs()
    q, k, v = bf(d["q"]), bf(d["k"]), bf(d["v"])
    op = torch.empty((1, 2048, 8, 128), dtype=torch.float32, device=dev)
    wsp = torch.empty(max(1, inv.inv_attention_prefill_workspace_bytes(1, 2048, 0, 8, 128)), dtype=torch.uint8, device=dev)
    def pre4():
        for _ in range(4):
            inv.inv_attention_prefill(q, k, v, out=op, ws=wsp)
    t = timeit(pre4) / 4
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
    # every position's decode row against the prefill row, and the prefill of the first 1024
    # rows (a different grid) against the same rows of the full prefill
    dall = torch.empty((2048, 8, 128), dtype=torch.float32, device=dev)
    for tt in range(2048):
        inv.inv_attention_decode(q[:, tt], k, v, posd[tt:tt + 1], out=dall[tt:tt + 1], ws=ws)
    half = inv.inv_attention_prefill(q[:, :1024].contiguous(), k, v)
    out(config="C2", bitwise_prefill_vs_decode=match(dall, op[0]), positions=2048,
        bitwise_prefill_1024_rows_vs_2048=match(half[0], op[0, :1024]))
# ---- C3: GEMM, weights cold (rotating copies > the 256 MB last-level cache)
if "C3" in SECTIONS:
    for (n, kk) in ((4096, 4096), (14336, 4096), (4096, 14336)):
        dd = synth.c3_inputs(n=n, k=kk, rows=512, seed_w=synth.SEEDS["c3_wdown"] if kk == 14336 else None,
                             seed_x=synth.SEEDS["c3_xdown"] if kk == 14336 else None)
        X = f32(dd["x"]); W0 = bf(dd["w"])
        ncp = max(2, int(600e6 // (n * kk * 2)) + 1)
        Ws = [W0] + [W0.clone() for _ in range(ncp - 1)]
        c3out = {}
        for M in (1, 3, 16, 64, 257, 512):
            Y = torch.empty((M, n), dtype=torch.float32, device=dev)
            ctr = [0]
            Xm = X[:M]
            def g():
                for _ in range(8):
                    inv.inv_fixed_order_gemm(Xm, Ws[ctr[0] % len(Ws)], out=Y); ctr[0] += 1
            t = timeit(g, reps=12) / 8
            by = n * kk * 2 + 4 * M * kk + 4 * M * n
            out(config="C3", N=n, K=kk, M=M, us=round(t * 1e6, 1), tflops=round(2 * M * n * kk / t / 1e12, 2),
                hbm_gbs=round(by / t / 1e9, 1), frac_hbm=round(by / t / 1e9 / HBM, 3), frac_fp32=round(2 * M * n * kk / t / 157.3e12, 3))
            c3out[M] = Y.clone()
        perm = torch.from_numpy(synth.permutation(7400, 512).astype(np.int64)).to(dev)
        shuf = inv.inv_fixed_order_gemm(X[perm].contiguous(), W0)
        out(config="C3", N=n, K=kk, bitwise_rows_vs_m512={M: match(c3out[M], c3out[512][:M]) for M in c3out},
            bitwise_shuffled_rows=match(shuf, c3out[512][perm]))
        del Ws
# ---- C4: LM head hidden 4096, vocab 128256, B = 1 .. 256
if "C4" in SECTIONS:
    d = synth.c4_inputs()
    H, W, T = f32(d["h"]), bf(d["w"]), torch.from_numpy(np.ascontiguousarray(d["target"], np.int32)).to(dev)
    c4out = {}
    for B in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        ws = torch.empty(inv.inv_lmhead_workspace_bytes(B, 4096, 128256), dtype=torch.uint8, device=dev)
        r = inv.inv_lmhead_logprob_top2(H[:B], W, T[:B], 0.1, ws=ws)
        c4out[B] = {k: r[k].clone() for k in LMK}
        nrec = int(r["recomputed"].sum().item())
        def four():
            for _ in range(4):
                inv.inv_lmhead_logprob_top2(H[:B], W, T[:B], 0.1, ws=ws, out=r)
        t = timeit(four, reps=6) / 4
        wb = 1050673152
        by = wb * (2 if (nrec and B > 32) else 1) + B * 4096 * 4
        out(config="C4", batch=B, recomputed=nrec, us=round(t * 1e6, 1), tokens_per_s=round(B / t, 1),
            hbm_gbs=round(by / t / 1e9, 1), frac_hbm=round(by / t / 1e9 / HBM, 3),
            tflops=round(2 * 128256 * 4096 * (B + nrec) / t / 1e12, 2))
    out(config="C4", bitwise_rows_vs_b256={B: min(match(c4out[B][k], c4out[256][k][:B]) for k in LMK) for B in c4out})
# ---- C5: decode steps of the 4-layer decoder at a 32k context, batch 1 .. 64 (graph replay;
# KV caches filled with seeded random values, every row at its own position near 32k)
if "C5" in SECTIONS:
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
    K5 = 4
    for B in (1, 4, 16, 64):
        run = dec5.decode_graph_steps(K5, B)
        tok = torch.randint(0, V5, (K5, B), dtype=torch.int32, device=dev, generator=g5)
        tgt = torch.randint(0, V5, (K5, B), dtype=torch.int32, device=dev, generator=g5)
        pos = torch.tensor([[T5 - 20 - 5 * b + k for b in range(B)] for k in range(K5)], dtype=torch.int32, device=dev)
        r = run(tok, pos, tgt)
        nrec = int(r[-1]["recomputed"].sum().item())
        t = timeit(lambda: run(tok, pos, tgt), reps=10) / K5
        kv = L5 * 2 * cfg["hkv"] * cfg["d"] * 4 * int((pos[-1] + 1).sum().item())
        by = body_w + head_w * (2 if (nrec and B > 32) else 1) + kv
        out(config="C5", op="decode", context=T5, batch=B, recomputed=nrec, ms_per_step=round(t * 1e3, 3),
            tokens_per_s=round(B / t, 1), hbm_gbs=round(by / t / 1e9, 1), frac_hbm=round(by / t / 1e9 / HBM, 3))
print("done", flush=True)
