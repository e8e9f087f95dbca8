"""Cross-precision greedy agreement on the Llama-shaped decoder (hidden 4096, 32/8 heads of
128, FFN 14336, vocabulary 128256, 4 layers; random-init BF16 weights, seeded synthetic
prompts), run on the library's kernels, plus the timings that go with it.

Policies: activation storage "fp32" (LayerCast), "bf16" or "fp16" for the body, and the
LM-head recompute threshold tau: 0 (BF16-input head only), 0.1 (selective FP32 recompute),
inf (FP32 head for every row).  "FP32" below is fp32 storage with tau = inf: with weights
that are BF16 values, that is the full-FP32 computation of the same model.

Prints one JSON object per line:
  * kind "pair": two policies compared on the same prompts (exact agreement, divergence
    index, flips versus margin; see invariant_numerics_amd.agreement);
  * kind "batch_invariance": a policy run with all prompts in one batch and prompt by prompt;
  * kind "margins": the histogram of the FP32 run's top-2 margins;
  * kind "decode_step": eager decode time per step of every storage policy at the harness
    batch, and graph-replayed LayerCast greedy decoding at B = 1, 2, 4, 8 with tau 0 and 0.1
    (the latency cost of selective recompute, with the share of steps that recomputed);
  * kind "round_kernel": the storage-rounding kernel's bandwidth on a 1 GiB tensor.
Usage: python bench_agreement.py [--prompts 16] [--prompt-len 32] [--steps 64]
"""
import argparse
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
import invariant_numerics_amd as inv  # noqa: E402
from invariant_numerics_amd import agreement  # noqa: E402
from invariant_numerics_amd.decoder import Decoder  # noqa: E402

PROMPT_SEED = 6001


def out(**k):
    print(json.dumps(k), flush=True)


def events():
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def timed_greedy(dec, prompts, steps):
    a, b = events()
    torch.cuda.synchronize()
    a.record()
    r = agreement.greedy(dec, prompts, steps)
    b.record()
    torch.cuda.synchronize()
    return r, a.elapsed_time(b) * 1e-3


def graph_greedy(dec, prompts, steps):
    """Greedy decoding with one captured decode step replayed per token (top-1 fed back on
    the device).  Returns (seconds for the decode steps, recomputed flags [B, steps])."""
    B, P = prompts.shape
    dev = prompts.device
    dec.prefill(prompts[:, :P - 1].contiguous())
    step = dec.decode_graph(B)
    tok = prompts[:, P - 1].contiguous()
    tgt = torch.zeros(B, dtype=torch.int32, device=dev)
    pos = [torch.full((B,), P - 1 + s, dtype=torch.int32, device=dev) for s in range(steps)]
    flags = []
    a, b = events()
    torch.cuda.synchronize()
    a.record()
    for s in range(steps):
        r = step(tok, pos[s], tgt)
        tok = r["top1"].clone()
        flags.append(r["recomputed"].clone())
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e-3, torch.stack(flags, 1).cpu().numpy()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--prompts", type=int, default=16)
    ap.add_argument("--prompt-len", type=int, default=32)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--timing-steps", type=int, default=48)
    args = ap.parse_args()
    if not torch.cuda.is_available():
        sys.exit("bench_agreement.py needs a GPU (the decoder runs the HIP kernels only)")
    dev = torch.device("cuda:0")
    cfg = dict(synth.C5)
    B, P, S = args.prompts, args.prompt_len, args.steps
    tmax = P + max(S, args.timing_steps)
    print("[step] building the model", flush=True)
    model = synth.decoder_model(cfg, tmax)
    prompts = torch.from_numpy(synth.tokens(PROMPT_SEED, B, P, cfg["vocab"])).to(dev)
    config = dict(workload="greedy continuation, Llama-shaped decoder 4 layers, hidden 4096, "
                  "vocab 128256, random-init", prompts=B, prompt_len=P, steps=S)

    decs = {}
    runs = {}
    secs = {}
    for act in ("fp32", "bf16", "fp16"):
        print("[step] decoder", act, flush=True)
        decs[act] = Decoder(model, device=dev, batch=B, tmax=tmax, act=act)
        for tau in ((0.0, 0.1, np.inf) if act == "fp32" else (0.0, 0.1)):
            decs[act].tau = float(np.float32(tau))
            print("[step] greedy", act, tau, flush=True)
            runs[(act, tau)], secs[(act, tau)] = timed_greedy(decs[act], prompts, S)

    def name(p):
        act, tau = p
        if act == "fp32":
            return {0.0: "LayerCast", 0.1: "LayerCast+recompute", np.inf: "FP32"}[tau]
        return "%s-body%s" % (act.upper(), "+recompute" if tau else "")

    pairs = [(("bf16", 0.0), ("fp16", 0.0)), (("bf16", 0.1), ("fp16", 0.1)),
             (("fp32", np.inf), ("bf16", 0.0)), (("fp32", np.inf), ("bf16", 0.1)),
             (("fp32", np.inf), ("fp16", 0.0)), (("fp32", np.inf), ("fp16", 0.1)),
             (("fp32", np.inf), ("fp32", 0.0)), (("fp32", np.inf), ("fp32", 0.1))]
    for pa, pb in pairs:
        r = agreement.compare(runs[pa], runs[pb])
        out(kind="pair", a=name(pa), b=name(pb), config=config, **r)
    out(kind="margins", run="FP32", config=config, **agreement.margin_histogram(runs[("fp32", np.inf)]))

    # batch composition: the first four prompts one by one against the batch-of-B run
    for act in ("fp32", "bf16", "fp16"):
        tau = 0.1
        decs[act].tau = float(np.float32(tau))
        same = True
        for i in range(4):
            one = agreement.greedy(decs[act], prompts[i:i + 1].contiguous(), S)
            for k in agreement.OUT_KEYS:
                x, y = np.ascontiguousarray(one[k][0]), np.ascontiguousarray(runs[(act, tau)][k][i])
                same &= bool(np.array_equal(x.view(np.uint8), y.view(np.uint8)))
        out(kind="batch_invariance", policy=name((act, tau)), batch_sizes=[B, 1], prompts_checked=4,
            bitwise_identical=same)

    for (act, tau), t in secs.items():
        out(kind="decode_step", mode="eager", policy=name((act, tau)), batch=B,
            ms_per_step=round(t / S * 1e3, 3), note="includes the prompt prefill")

    # selective recompute: latency at small batch, graph-replayed decode (LayerCast body)
    dec = decs["fp32"]
    for b in (1, 2, 4, 8):
        res = {}
        for tau in (0.0, 0.1):
            dec.tau = float(np.float32(tau))
            graph_greedy(dec, prompts[:b].contiguous(), 4)        # warm-up and capture
            t, fl = graph_greedy(dec, prompts[:b].contiguous(), args.timing_steps)
            res[tau] = (t, fl)
        t0, t1 = res[0.0][0], res[0.1][0]
        fl = res[0.1][1]
        out(kind="decode_step", mode="graph", policy="LayerCast", batch=b, steps=args.timing_steps,
            ms_per_step_tau0=round(t0 / args.timing_steps * 1e3, 4),
            ms_per_step_tau01=round(t1 / args.timing_steps * 1e3, 4),
            recompute_overhead=round(t1 / t0 - 1.0, 4),
            rows_recomputed=round(float(fl.mean()), 4),
            steps_with_recompute=round(float(fl.any(axis=0).mean()), 4))
    del decs, dec
    torch.cuda.empty_cache()

    # storage-rounding kernel: 1 GiB of FP32, 8 algorithmic bytes per element
    n = 1 << 28
    x = torch.randn(n // 4096, 4096, device=dev)
    y = torch.empty_like(x)
    for fmt in ("bf16", "fp16"):
        for _ in range(2):
            inv.inv_round_activations(x, fmt, out=y)
        ts = []
        for _ in range(10):
            a, b = events()
            a.record()
            inv.inv_round_activations(x, fmt, out=y)
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        t = float(np.median(ts))
        gbs = 8.0 * n / t / 1e9
        out(kind="round_kernel", fmt=fmt, elements=n, us=round(t * 1e6, 1), gb_per_s=round(gbs, 1),
            frac_of_8tbs=round(gbs / 8000.0, 3))


if __name__ == "__main__":
    main()
