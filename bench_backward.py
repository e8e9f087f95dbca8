"""Throughput of the fixed-order matmul backward (dX over the outputs, dW over the tokens)
for the four projections of the 4-layer hidden-4096 decoder (QKV 6144x4096, O 4096x4096,
W1||W3 28672x4096, W2 4096x14336) over one 16384-token block, with the forward beside it.

Seeded synthetic operands (dY ~ N(0, 0.01^2), X ~ N(0, 1), W ~ N(0, 0.02^2) in BF16),
resident in HBM; each figure is the median of HIP-event-bracketed calls on the current
stream.  Prints one JSON object per projection and gradient, with TFLOP/s (2 M N K flops
per gradient) and the fraction of the 157.3 TFLOP/s FP32 matrix peak.
The LM head of a policy-gradient step is timed over 1024 tokens: the logit gradient
(inv_lmhead_logit_grad), the hidden-state gradient and the head's weight gradient
(inv_gemm_backward on it); 2 B V K flops each.
Usage: python bench_backward.py [--tokens 16384] [--head-tokens 1024]
"""
import argparse
import json
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import numpy as np  # noqa: E402
import torch  # noqa: E402

import invariant_numerics_amd as inv  # noqa: E402

PEAK = 157.3e12


def timeit(fn, reps=5, warm=1):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) * 1e-3)
    return float(np.median(ts))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--tokens", type=int, default=16384)
    ap.add_argument("--head-tokens", type=int, default=1024)
    args = ap.parse_args()
    if not torch.cuda.is_available():
        sys.exit("bench_backward.py needs a GPU (the library runs HIP kernels only)")
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(8800)
    M = args.tokens
    for name, N, K in (("qkv", 6144, 4096), ("o", 4096, 4096), ("w13", 28672, 4096), ("w2", 4096, 14336)):
        X = torch.randn(M, K, device=dev, generator=g)
        dY = torch.randn(M, N, device=dev, generator=g) * 0.01
        W = (torch.randn(N, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)
        dX = torch.empty(M, K, device=dev)
        dW = torch.empty(N, K, device=dev)
        Y = torch.empty(M, N, device=dev)
        ws = torch.empty(inv.inv_gemm_backward_workspace_bytes(M, N, K), dtype=torch.uint8, device=dev)
        fl = 2.0 * M * N * K
        t_f = timeit(lambda: inv.inv_fixed_order_gemm(X, W, out=Y))
        t_x = timeit(lambda: inv.inv_gemm_backward(dY, None, W, dw=False, out_dx=dX, ws=ws))
        t_w = timeit(lambda: inv.inv_gemm_backward(dY, X, W, dx=False, out_dw=dW))
        for what, t in (("forward", t_f), ("dX", t_x), ("dW", t_w)):
            print(json.dumps(dict(projection=name, tokens=M, N=N, K=K, op=what, ms=round(t * 1e3, 3),
                                  tflops=round(fl / t / 1e12, 1), frac_fp32_peak=round(fl / t / PEAK, 3))),
                  flush=True)
        del X, dY, W, dX, dW, Y, ws
        torch.cuda.empty_cache()
    # LM head of a policy-gradient step over a block of tokens: logit gradient (FP32 logits,
    # fixed-order softmax, coef * ([v == t] - p)), then the hidden-state gradient (sum over
    # the 128256 logits) and the head's weight gradient (sum over the tokens)
    B, K, V = args.head_tokens, 4096, 128256
    H = torch.randn(B, K, device=dev, generator=g)
    W = (torch.randn(V, K, device=dev, generator=g) * 0.02).to(torch.bfloat16)
    tgt = torch.randint(0, V, (B,), dtype=torch.int32, device=dev, generator=g)
    coef = torch.randn(B, device=dev, generator=g)
    G = torch.empty(B, V, device=dev)
    dH = torch.empty(B, K, device=dev)
    dW = torch.empty(V, K, device=dev)
    gws = torch.empty(inv.inv_lmhead_logit_grad_workspace_bytes(B, K, V), dtype=torch.uint8, device=dev)
    bws = torch.empty(inv.inv_gemm_backward_workspace_bytes(B, V, K), dtype=torch.uint8, device=dev)
    fl = 2.0 * B * V * K
    t_g = timeit(lambda: inv.inv_lmhead_logit_grad(H, W, tgt, coef, out=G, ws=gws))
    t_x = timeit(lambda: inv.inv_gemm_backward(G, None, W, dw=False, out_dx=dH, ws=bws))
    t_w = timeit(lambda: inv.inv_gemm_backward(G, H, W, dx=False, out_dw=dW))
    for what, t in (("logit_grad", t_g), ("dH", t_x), ("dW_head", t_w)):
        print(json.dumps(dict(projection="lm_head", tokens=B, N=V, K=K, op=what, ms=round(t * 1e3, 3),
                              tflops=round(fl / t / 1e12, 1), frac_fp32_peak=round(fl / t / PEAK, 3))),
              flush=True)


if __name__ == "__main__":
    main()
