"""Benchmark: batch-invariant token scoring with the 4-layer Llama-8B-shaped decoder.

One step = score one batch of synthetic sequences end to end through the whole hot path:
embedding gather, per layer RMSNorm -> QKV fixed-order GEMM -> RoPE + KV append ->
chunked causal attention -> O GEMM + residual -> RMSNorm -> W1||W3 GEMM -> SwiGLU ->
W2 GEMM + residual; final RMSNorm; LM head (BF16 pass, log-softmax, top-2, margin) with
selective FP32 recompute of rows whose margin < 0.1.  Inputs (weights, tokens) are
resident in HBM before the timed region.  value = scored tokens / s = B * (T - 1) / step.

Also printed in the same JSON line:
  roofline      the dominant kernel (the body projections' FP32-MFMA GEMM), timed
                with HIP events on its launch stream inside the timed steps;
  cpu_baseline  the CPU oracle on bounded samples of the same workload (a 64-token sequence
                at full width on all host threads, a 4-token one on one thread), scaled to
                tokens / s, with the per-token work of the sample and of the 32k workload;
  bitwise       match rates: repeated steps; prefill vs token-by-token decode at the end of
                the long context; the same rows across batch sizes 1..64 (the LM head, and a
                decode step at a 32k context); the GPU against the oracle on the CPU sample
                and, at the timed launch configurations, on sampled outputs of each timed
                kernel (seeded inputs of the same shapes).

Usage: python bench.py [--gpus 1] [--steps 3] [--warmup 1] [--batch 1] [--seq 32768]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# up to this many rows the LM head computes the FP32 (recompute) logits in the same sweep over
# the vocabulary weights as the primary ones, so a recomputed row adds no weight read
LM_SHARED_SWEEP_MAX_B = 32
FP32_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix (MFMA) peak: 256 CU x 2.4 GHz x 256 flop/clk


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--seq", type=int, default=32768)
    ap.add_argument("--block", type=int, default=16384, help="token rows per prefill block")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="before the timed steps, copy 1 GiB device to device once (untimed): the "
                         "reference dispatch for scaling HBM byte counters in profiler runs")
    return ap.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_128x256_c5_prefill_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "invariant_numerics_amd", "csrc", "gemm.hip")


GEMM_KERNEL_HEAD = "template <int BM, int BN, int WGM, int WGN, int ROLE>\n__global__"


def gemm_kernel_sha():
    """SHA-256 of the tiled GEMM kernel's own source text (its template line to its closing
    brace), so that edits elsewhere in the file do not void the recorded counters."""
    import hashlib
    src = open(GEMM_SOURCE).read()
    i = src.index(GEMM_KERNEL_HEAD)
    j = src.index("\n}\n", i) + 3
    return hashlib.sha256(src[i:j].encode()).hexdigest()


def measured_traffic(block):
    """HBM bytes per launch of the body-projection GEMM from the profiler counter runs recorded
    under profiles/ (FETCH_SIZE + WRITE_SIZE, scaled by a 1 GiB copy), or None when the kernel
    source has changed since they were taken or they were taken at another token block."""
    try:
        vals = dict(line.split(": ", 1) for line in open(TRAFFIC_FILE).read().splitlines() if ": " in line)
        sha = gemm_kernel_sha()
        if vals.get("gemm_kernel_sha256", "").strip() != sha:
            return None
        if int(vals.get("token_block", "0")) != block:
            return None
        return int(vals["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None

BATCHES = (1, 2, 4, 8, 16, 32, 64)
LM_KEYS = ("logprob", "margin", "top1", "top2", "recomputed")


def _rate(a, b):
    import torch
    a = a.contiguous().view(torch.int32) if a.dtype == torch.float32 else a
    b = b.contiguous().view(torch.int32) if b.dtype == torch.float32 else b
    return (a == b).float().mean().item()


def across_batch(dec, model, cfg, dev, T):
    """The same rows at every batch size in BATCHES: (1) 64 LM-head rows run as 64 / B calls of
    B rows; (2) one decode step at position T - 1 of a 32k context for sequences 0..B-1 (seeded
    random KV caches of 64 sequences).  Each B's rows are compared with the B = 64 rows."""
    import torch
    import synth
    from invariant_numerics_amd import binding as inv
    from invariant_numerics_amd.decoder import Decoder
    out = {}
    h = torch.from_numpy(synth.normal(15100, (64, cfg["hidden"]))).to(dev)
    tg = torch.from_numpy(synth.uniform_int(15101, (64,), cfg["vocab"])).to(dev)
    full = inv.inv_lmhead_logprob_top2(h, dec.whead, tg, 0.1)
    lm = {}
    for B in BATCHES:
        parts = [inv.inv_lmhead_logprob_top2(h[s:s + B], dec.whead, tg[s:s + B], 0.1) for s in range(0, 64, B)]
        lm[str(B)] = min(_rate(torch.cat([p[k] for p in parts]), full[k]) for k in LM_KEYS)
    out["lmhead_rows64"] = lm
    nb = max(BATCHES)
    dd = Decoder.__new__(Decoder)
    dd.__dict__.update(dec.__dict__)
    dd.batch = nb
    g = torch.Generator(device=dev)
    g.manual_seed(15102)
    dd.kc = [torch.randn((nb, cfg["hkv"], T, cfg["d"]), generator=g, device=dev) for _ in range(cfg["layers"])]
    dd.vc = [torch.randn((nb, cfg["hkv"], T, cfg["d"]), generator=g, device=dev) for _ in range(cfg["layers"])]
    dd.gemm_events = None
    tok = torch.from_numpy(synth.uniform_int(15103, (nb,), cfg["vocab"])).to(dev)
    tgt = torch.from_numpy(synth.uniform_int(15104, (nb,), cfg["vocab"])).to(dev)
    pos = torch.full((nb,), T - 1, dtype=torch.int32, device=dev)
    ref = dd.decode_step(tok, pos, tgt)
    dec_rates = {}
    for B in BATCHES:
        r = dd.decode_step(tok[:B].contiguous(), pos[:B].contiguous(), tgt[:B].contiguous())
        dec_rates[str(B)] = min(_rate(r[k], ref[k][:B]) for k in LM_KEYS)
    out["decode_32k"] = dec_rates
    out["decode_context"] = T - 1
    # graph-replayed decode steps at larger batches on the same caches (timing only): four
    # steps at the same position per graph, as in the decode timing of the main check
    timing = {}
    H, F, V, L = cfg["hidden"], cfg["ffn"], cfg["vocab"], cfg["layers"]
    QKV = (cfg["hq"] + 2 * cfg["hkv"]) * cfg["d"]
    weights = L * 2 * (QKV * H + H * cfg["hq"] * cfg["d"] + 2 * F * H + H * F) + 2 * V * H
    KS_ = 4
    for B in (16, 64):
        grun = dd.decode_graph_steps(KS_, B)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(4)]
        args_ = tuple(x[:B].contiguous().unsqueeze(0).repeat(KS_, 1) for x in (tok, pos, tgt))
        grun(*args_)
        for a_, b_ in ev:
            a_.record()
            r = grun(*args_)
            b_.record()
        torch.cuda.synchronize()
        nrec = int(r[-1]["recomputed"].sum().item())
        sec = float(np.median([a_.elapsed_time(b_) for a_, b_ in ev])) * 1e-3 / KS_
        kv = L * 2 * cfg["hkv"] * T * cfg["d"] * 4 * B
        nbytes = weights + kv + (2 * V * H if (nrec and B > LM_SHARED_SWEEP_MAX_B) else 0)
        timing[str(B)] = dict(ms_per_step=round(sec * 1e3, 3), tokens_per_s=round(B / sec, 1),
                              algorithmic_bytes_per_step=float(nbytes),
                              hbm_frac=round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4))
        del grun
    out["decode_32k_graph_timing"] = timing
    del dd
    torch.cuda.synchronize()
    return out


def kernel_parity(orc, model, cfg, dev, T, block):
    """Each kernel the timed steps run, launched at the timed configuration (16384-row token
    blocks, a 32k context, one-row decode) on seeded synthetic inputs of the same shapes,
    against the oracle on sampled outputs.  Returns {kernel: [matching words, words]}."""
    import torch
    import synth
    from invariant_numerics_amd import binding as inv
    H, F, V, Hq, Hkv, D = (cfg[k] for k in ("hidden", "ffn", "vocab", "hq", "hkv", "d"))
    lay = model["layers"][0]
    res = {}

    def rec(name, got, want):
        g = np.ascontiguousarray(got)
        w = np.ascontiguousarray(want)
        if g.dtype == np.float32:
            g, w = g.view(np.uint32), w.view(np.uint32)
        same, tot = res.get(name, (0, 0))
        res[name] = (same + int((g == w).sum()), tot + int(g.size))

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    def dev_f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    M = block
    rows = np.array(sorted({0, 1, 15, 63, 64, 127, 128, 4095, 8191, M - 65, M - 1}))
    cols = lambda n: np.array(sorted(set(synth.permutation(15200 + n, n)[:48].tolist()) | {0, 255, n - 1}))
    # body projections on the 128 x 256 tile: QKV (plain), W2 with the residual, W1||W3 gated
    X = synth.normal(15201, (M, H))
    Xd = dev_f32(X)
    w = lay["wqkv"]
    nm = inv.inv_kernel_route("gemm", M, w.shape[0])
    c = cols(w.shape[0])
    rec(nm, inv.inv_fixed_order_gemm(Xd, dev_bf16(w)).cpu().numpy()[rows][:, c], orc.gemm(X[rows], w[c]))
    w13 = lay["w13"]
    wi = np.empty_like(w13)
    wi[0::2], wi[1::2] = w13[:F], w13[F:]
    nm = inv.inv_kernel_route("gated_gemm", M, 2 * F)
    c = cols(F)
    got = inv.inv_gated_gemm(Xd, dev_bf16(wi)).cpu().numpy()[rows][:, c]
    rec(nm, got, orc.swiglu(orc.gemm(X[rows], w13[c]), orc.gemm(X[rows], w13[F + c])))
    del Xd
    Xf = synth.normal(15202, (M, F))
    R = synth.normal(15203, (M, H))
    w = lay["w2"]
    nm = inv.inv_kernel_route("gemm", M, H) + " +R"
    c = cols(H)
    got = inv.inv_fixed_order_gemm(dev_f32(Xf), dev_bf16(w), R=dev_f32(R)).cpu().numpy()[rows][:, c]
    rec(nm, got, (R[rows][:, c] + orc.gemm(Xf[rows], w[c])).astype(np.float32))
    del Xf, R
    torch.cuda.empty_cache()
    # attention prefill: the second 16384-row block of a 32k sequence (FP32 cache)
    q = synth.normal(15204, (1, M, Hq, D))
    k = synth.normal(15205, (1, Hkv, T, D))
    v = synth.normal(15206, (1, Hkv, T, D))
    kd, vd = dev_f32(k), dev_f32(v)
    q0 = T - M
    got = inv.inv_attention_prefill(dev_f32(q), kd, vd, q_start=q0).cpu().numpy()
    nm = inv.inv_kernel_route("attention_prefill", Hq, M).replace("DT", "1")
    for r in rows[::2]:
        rec(nm, got[:, r:r + 1], orc.attention(q[:, r:r + 1], k, v, q_start=q0 + int(r)))
    # decode attention at the end of the context
    pos = np.array([T - 2], np.int32)
    qd = synth.normal(15207, (1, Hq, D))
    got = inv.inv_attention_decode(dev_f32(qd), kd, vd, torch.from_numpy(pos).to(dev)).cpu().numpy()
    rec("attn_decode_partial_kernel<1,4> + attn_decode_merge_kernel", got[0],
        orc.attention(qd[None], k, v, q_start=int(pos[0]))[0, 0])
    del kd, vd
    # decode-step projections at one row (the VALU GEMV): QKV and W1||W3 with the RMSNorm in
    # their prologue (QKV with RoPE and the KV append), O plain, W2 below
    x1 = synth.normal(15208, (1, H))
    gam = synth.to_bf16_bits(np.float32(1.0) + synth.normal(15212, (H,), 0.1))
    n1 = orc.rmsnorm(x1, gam)
    w = lay["wqkv"]
    nm = inv.inv_kernel_route("gemm", 1, w.shape[0]).replace("<1,0,", "<1,3,") + " + RMSNorm prologue, RoPE, KV append"
    tm, p1 = 64, np.array([37], np.int32)
    cos_t, sin_t = synth.rope_tables(tm, D, cfg["theta"])
    qo = torch.zeros((1, Hq, D), device=dev)
    kc = torch.zeros((1, Hkv, tm, D), device=dev)
    vc = torch.zeros((1, Hkv, tm, D), device=dev)
    inv.inv_rmsnorm_qkv_rope_kv_append(dev_f32(x1), dev_bf16(gam), dev_bf16(w), Hq, Hkv, D,
                                       torch.zeros(1, dtype=torch.int32, device=dev), torch.from_numpy(p1).to(dev),
                                       dev_f32(cos_t), dev_f32(sin_t), qo, kc, vc)
    qkv = orc.gemm(n1, w)
    rec(nm, qo.cpu().numpy(), orc.rope(qkv[:, :Hq * D].reshape(1, Hq, D), p1, cos_t, sin_t))
    rec(nm, kc.cpu().numpy()[0, :, 37], orc.rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(1, Hkv, D), p1, cos_t,
                                                  sin_t)[0])
    rec(nm, vc.cpu().numpy()[0, :, 37], qkv[:, (Hq + Hkv) * D:].reshape(Hkv, D))
    w = lay["wo"]
    nm = inv.inv_kernel_route("gemm", 1, w.shape[0])
    rec(nm, inv.inv_fixed_order_gemm(dev_f32(x1), dev_bf16(w)).cpu().numpy(), orc.gemm(x1, w))
    nm = inv.inv_kernel_route("gated_gemm", 1, 2 * F) + " + RMSNorm prologue"
    rec(nm, inv.inv_rmsnorm_gemm(dev_f32(x1), dev_bf16(gam), dev_bf16(wi), gated=True).cpu().numpy(),
        orc.swiglu(orc.gemm(n1, w13[:F]), orc.gemm(n1, w13[F:])))
    x1f = synth.normal(15209, (1, F))
    nm = inv.inv_kernel_route("gemm", 1, H) + " (K 14336)"
    rec(nm, inv.inv_fixed_order_gemm(dev_f32(x1f), dev_bf16(lay["w2"])).cpu().numpy(), orc.gemm(x1f, lay["w2"]))
    # LM head: one decode row, and sampled rows of a 16384-row block
    wh = dev_bf16(model["whead"])
    hb = synth.normal(15210, (M, H))
    tg = synth.uniform_int(15211, (M,), V)
    for B, rr in ((1, np.array([0])), (M, rows[::3])):
        r = inv.inv_lmhead_logprob_top2(dev_f32(hb[:B]), wh, torch.from_numpy(tg[:B]).to(dev), 0.1)
        want = orc.lmhead(hb[rr], model["whead"], tg[rr])
        nm = "lmhead: " + inv.inv_kernel_route("lmhead_gemm", B, V) + " + reductions"
        for key in LM_KEYS:
            rec(nm, r[key].cpu().numpy()[rr], want[key])
    torch.cuda.synchronize()
    return {k: [a, b] for k, (a, b) in res.items()}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def per_token_gflop(cfg, T, recomputed):
    """Average algorithmic GFLOP per scored token of a T-token sequence: body projections,
    LM head (primary pass plus the recomputed fraction), causal attention (4 D flops per
    query-key pair and head, averaged over positions)."""
    H, F, V, Hq, Hkv, D, L = (cfg[k] for k in ("hidden", "ffn", "vocab", "hq", "hkv", "d", "layers"))
    body = 2 * L * ((Hq + 2 * Hkv) * D * H + H * Hq * D + 2 * F * H + H * F)
    head = 2 * V * H * (1 + recomputed)
    attn = L * Hq * 4 * D * (T + 1) / 2.0
    return (body + head + attn) / 1e9


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows are independent, so N GPUs would each score their own sequences). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    from invariant_numerics_amd import binding as inv
    from invariant_numerics_amd.decoder import Decoder

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cfg = dict(synth.C5)
    cfg["layers"] = args.layers
    B, T = args.batch, args.seq
    t0 = time.time()
    log("generating synthetic model", cfg)
    model = synth.decoder_model(cfg, T)
    toks = synth.tokens(synth.SEEDS["c5_tok"], B, T, cfg["vocab"])
    log("model ready in %.1fs" % (time.time() - t0))
    dec = Decoder(model, device=dev, batch=B, tmax=T)
    td = torch.from_numpy(toks).to(dev)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed steps
    def step():
        return dec.prefill(td, block=args.block)

    for i in range(args.warmup):
        log("warmup", i)
        out = step()
    torch.cuda.synchronize()
    if args.calib_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 1 GiB read + 1 GiB written")
    rec = []
    dec.gemm_events = rec
    outs = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        outs.append(step())
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    dec.gemm_events = None
    ms = elapsed / args.steps * 1e3
    scored = B * (T - 1)
    value = scored * args.steps / elapsed
    log("step %.1f ms, %.0f scored tok/s" % (ms, value))

    # dominant kernel: body projections, HIP events on the launch stream
    durs = np.array([s.elapsed_time(e) for s, e, _, _ in rec]) * 1e-3  # seconds
    flops = np.array([f for _, _, f, _ in rec], np.float64)
    achieved = float(flops.sum() / durs.sum()) / 1e12
    gemm_share = float(durs.sum() / elapsed)
    default_workload = (B == 1 and T == 32768 and args.layers == 4)
    roof = dict(bound="mfma", kernel="gemm_mfma_kernel<128,256,2,4,0|2> (the four body projections; W1||W3 with the gated SwiGLU epilogue; FP32 matrix cores, 32x32x2)",
                achieved=round(achieved, 3),
                peak=FP32_PEAK_TFLOPS, unit="TFLOP/s", frac=round(achieved / FP32_PEAK_TFLOPS, 4),
                traffic=measured_traffic(args.block) if default_workload else None,
                traffic_unit="bytes per launch (HBM read + write, counter-measured)",
                algorithmic_bytes_per_launch=float(np.mean([b for _, _, _, b in rec])) if rec else None,
                launches=int(len(rec)), avg_launch_us=round(float(durs.mean()) * 1e6, 2),
                avg_flops_per_launch=float(flops.mean()), share_of_step=round(gemm_share, 3))
    recomputed = float(outs[-1]["recomputed"].float().mean().item())

    # ---------------------------------------------------------------- bitwise checks
    bitwise = {}
    decode = None
    if not args.no_check:
        keys = ("logprob", "margin", "top1", "top2", "recomputed")

        def rate(a, b):
            a = a.contiguous().view(torch.int32) if a.dtype == torch.float32 else a
            b = b.contiguous().view(torch.int32) if b.dtype == torch.float32 else b
            return (a == b).float().mean().item()

        bitwise["repeat_steps"] = min(rate(outs[0][k], outs[-1][k]) for k in keys)
        # prefill vs token-by-token decode on the last positions of the long context; the
        # decode steps are also timed (HBM-bound path: every weight byte and the whole KV
        # cache are read once per step)
        ndec = min(16, T - 1)
        p0 = T - 1 - ndec
        log("decode check: prefill %d tokens, then %d decode steps" % (p0, ndec))
        dd = Decoder.__new__(Decoder)
        dd.__dict__.update(dec.__dict__)
        dd.kc = [torch.zeros_like(k) for k in dec.kc]
        dd.vc = [torch.zeros_like(v) for v in dec.vc]
        dd.gemm_events = None
        if p0 > 0:
            dd.prefill(td[:, :p0 + 1].contiguous(), block=args.block)
        gstep = dd.decode_graph(B)      # one decode step captured as a HIP graph
        H, F, V, L = cfg["hidden"], cfg["ffn"], cfg["vocab"], cfg["layers"]
        QKV = (cfg["hq"] + 2 * cfg["hkv"]) * cfg["d"]
        body_w = L * 2 * (QKV * H + H * cfg["hq"] * cfg["d"] + 2 * F * H + H * F)
        head_w = 2 * V * H
        steps_t = list(range(p0, T - 1))
        pos_all = [torch.full((B,), t, dtype=torch.int32, device=dev) for t in steps_t]
        tok_all = [td[:, t].contiguous() for t in steps_t]
        tgt_all = [td[:, t + 1].contiguous() for t in steps_t]
        # device time: the steps are enqueued back to back (no host synchronisation between
        # them); events bracket each step's input copies and graph replay on the stream
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in steps_t]
        res = []
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(len(steps_t)):
            ev[i][0].record()
            r = gstep(tok_all[i], pos_all[i], tgt_all[i])
            ev[i][1].record()
            res.append({k: v.clone() for k, v in r.items()})
        torch.cuda.synchronize()
        host_s = (time.perf_counter() - t1) / len(steps_t)
        step_s = [s_.elapsed_time(e_) * 1e-3 for s_, e_ in ev]
        agree = []
        step_bytes = []
        for i, t in enumerate(steps_t):
            kv = L * 2 * cfg["hkv"] * (t + 1) * cfg["d"] * 4 * B
            nrec = int(res[i]["recomputed"].sum().item())
            head_sweeps = 2 if (nrec and B > LM_SHARED_SWEEP_MAX_B) else 1
            step_bytes.append(body_w + head_w * head_sweeps + kv)
            agree.append(min(rate(res[i][k], outs[-1][k][:, t]) for k in keys))
        bitwise["prefill_vs_decode"] = float(np.mean(agree))
        bitwise["prefill_vs_decode_positions"] = [p0, T - 2]
        # drop the first step (first touch of the decode path)
        ds = np.array(step_s[1:]) if len(step_s) > 1 else np.array(step_s)
        db = np.array(step_bytes[1:]) if len(step_bytes) > 1 else np.array(step_bytes)
        gbs = float(db.sum() / ds.sum()) / 1e9
        # the same steps as one graph of K steps: one replay runs them in order with one launch
        # and one set of input copies; its outputs must be the single-step graph's, bit for bit
        K = len(steps_t)
        mrun = dd.decode_graph_steps(K, B)
        tokK, posK, tgtK = torch.stack(tok_all), torch.stack(pos_all), torch.stack(tgt_all)
        rK = mrun(tokK, posK, tgtK)
        torch.cuda.synchronize()
        bitwise["multi_step_graph_vs_single_step"] = float(min(rate(rK[i][k], res[i][k]) for i in range(K) for k in keys))
        evm = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(5)]
        for a_, b_ in evm:
            a_.record()
            mrun(tokK, posK, tgtK)
            b_.record()
        torch.cuda.synchronize()
        msec = float(np.median([a_.elapsed_time(b_) for a_, b_ in evm])) * 1e-3 / K
        # the last timed replay's outputs as well (replays after the first must match too)
        bitwise["multi_step_graph_vs_single_step"] = min(
            bitwise["multi_step_graph_vs_single_step"],
            float(min(rate(rK[i][k], res[i][k]) for i in range(K) for k in keys)))
        mbytes = float(np.mean(step_bytes))
        decode = dict(context=p0, batch=B, steps=K, ms_per_step=round(msec * 1e3, 3),
                      tokens_per_s=round(B / msec, 2),
                      algorithmic_bytes_per_step=mbytes,
                      hbm_gbs=round(mbytes / msec / 1e9, 1), hbm_frac=round(mbytes / msec / 1e9 / HBM_PEAK_GBS, 4),
                      single_step_graph=dict(steps=int(len(ds)), ms_per_step=round(float(ds.mean()) * 1e3, 3),
                                             hbm_frac=round(gbs / HBM_PEAK_GBS, 4),
                                             host_ms_per_step=round(host_s * 1e3, 3)),
                      note="K consecutive decode steps (all layers + LM head incl. recompute pass) captured "
                           "as one HIP graph, replayed and timed with HIP events on the stream (median of 5 "
                           "replays, divided by K; the input copies of the K steps included); "
                           "single_step_graph: the same steps as K replays of a one-step graph, enqueued "
                           "back to back, each with its own input copies (first step dropped); bytes = "
                           "BF16 weights + FP32 KV cache read once (+ a second vocabulary sweep when a "
                           "row is recomputed and the batch exceeds 32 rows)")
        del dd
        # context for the decode fraction: a plain device copy (1 GiB read + 1 GiB written),
        # timed the same way
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        ce = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(3)]
        for a_, b_ in ce:
            a_.record()
            dst.copy_(src)
            b_.record()
        torch.cuda.synchronize()
        copy_s = min(a_.elapsed_time(b_) for a_, b_ in ce) * 1e-3
        decode["copy_gbs_read_plus_write"] = round(2 * (1 << 30) / copy_s / 1e9, 1)
        del src, dst

    if not args.no_check:
        log("across-batch check: B in %s" % (BATCHES,))
        bitwise["across_batch"] = across_batch(dec, model, cfg, dev, T)

    # ---------------------------------------------------------------- CPU baseline
    # (the only part of this script that runs the oracle: timing it on the host cores, and
    # comparing the GPU with it)
    cpu = None
    if not args.no_cpu:
        from oracle import oracle as orc
        orc.lib()
        n = args.cpu_tokens
        sample = toks[0, :n].copy()
        threads = orc.set_threads(0)
        log("cpu baseline: oracle on %d tokens at full width, %d threads" % (n, threads))
        tc = time.perf_counter()
        want = orc.decoder(sample, model)
        tcpu = time.perf_counter() - tc
        n1 = 4
        one = orc.set_threads(1)
        log("cpu baseline: oracle on %d tokens, %d thread" % (n1, one))
        tc = time.perf_counter()
        orc.decoder(sample[:n1].copy(), model)
        tcpu1 = time.perf_counter() - tc
        orc.set_threads(0)
        rec_frac = float(np.mean(want["recomputed"]))
        g_sample = per_token_gflop(cfg, n, rec_frac)
        g_sample1 = per_token_gflop(cfg, n1, rec_frac)
        g_work = per_token_gflop(cfg, T, recomputed)
        cpu = dict(value=round((n - 1) / tcpu, 3), unit="scored tokens/s", cores=threads, kind="oracle",
                   sample="one %d-token sequence through the same 4-layer full-width decoder and LM head "
                          "(hidden 4096, vocab 128256, selective recompute) on %d threads: %.1f s; "
                          "%.2f GFLOP per scored token against %.2f for the %d-token workload" %
                          (n, threads, tcpu, g_sample, g_work, T),
                   cpu_model=cpu_model(), host_cpus=os.cpu_count(),
                   single_thread=dict(value=round((n1 - 1) / tcpu1, 4), cores=one, tokens=n1,
                                      seconds=round(tcpu1, 2),
                                      gflop_per_token=round(g_sample1, 3)),
                   gflop_per_token_sample=round(g_sample, 3), gflop_per_token_workload=round(g_work, 3),
                   value_at_workload_cost=round((n - 1) / tcpu * g_sample / g_work, 3))
        if not args.no_check:
            g = Decoder(model, device=dev, batch=1, tmax=n).prefill(torch.from_numpy(sample[None]).to(dev))
            tot = 0
            same = 0
            for k, w in want.items():
                a = g[k][0].cpu().numpy()
                if a.dtype == np.float32:
                    a, w = a.view(np.uint32), w.view(np.uint32)
                same += int((a == w).sum())
                tot += a.size
            bitwise["vs_oracle"] = same / tot
            bitwise["vs_oracle_words"] = tot
            bitwise["vs_oracle_kernels"] = sorted({
                inv.inv_kernel_route("gemm", n, (cfg["hq"] + 2 * cfg["hkv"]) * cfg["d"]),
                inv.inv_kernel_route("gemm", n, cfg["hidden"]),
                inv.inv_kernel_route("gated_gemm", n, 2 * cfg["ffn"]),
                inv.inv_kernel_route("attention_prefill", cfg["hq"], n),
                inv.inv_kernel_route("lmhead_gemm", n, cfg["vocab"])})
            log("kernel parity at the timed launch configurations")
            kp = kernel_parity(orc, model, cfg, dev, T, args.block)
            bitwise["timed_kernels_vs_oracle"] = {k: round(a / b, 6) for k, (a, b) in kp.items()}
            bitwise["timed_kernels_vs_oracle_words"] = int(sum(b for _, b in kp.values()))

    line = dict(
        metric="scored tokens/s (batch-invariant) + % HBM/FLOP roofline; bitwise-match rate",
        value=round(value, 2), unit="scored tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 3), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="f32", data="synthetic",
        config=dict(workload="4-layer Llama-8B-shaped decoder, prefill scoring with selective FP32 "
                             "LM-head recompute", layers=cfg["layers"], hidden=cfg["hidden"],
                    q_heads=cfg["hq"], kv_heads=cfg["hkv"], head_dim=cfg["d"], ffn=cfg["ffn"],
                    vocab=cfg["vocab"], batch=B, seq_len=T, token_block=args.block, tau=0.1,
                    weights="bf16 storage, fp32 compute", recomputed_fraction=round(recomputed, 4)),
        roofline=roof, cpu_baseline=cpu, bitwise=bitwise, decode=decode)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
