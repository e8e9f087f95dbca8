"""Cross-precision greedy agreement on synthetic (random-init) models.

The same prompts are continued greedily under two numerical policies -- an activation
storage format for the decoder body ("fp32" = LayerCast, "bf16", "fp16") and an LM-head
recompute threshold tau (0 = low-precision head only, 0.1 = selective FP32 recompute,
inf = FP32 head for every row) -- and the continuations are compared token by token:

  * exact agreement: the share of prompts whose continuations are identical;
  * divergence index: the first generated position at which the two runs pick different
    tokens (the reproducibility study's Divergence Index; ``steps`` when they never differ);
  * flip versus margin: at every step before the divergence both runs have the same prefix.
    With (a1, a2) run A's top two candidates and m_A = z_a1 - z_a2 >= 0 its margin, run B's
    gap between the same two candidates is g_B = +m_B or -m_B (B's margin, signed by whether
    B ranks them the same way); d = m_A - g_B is the directional perturbation between the runs
    along the top-two direction.  B flips the token exactly when g_B < 0, i.e. when d exceeds
    the margin ("Greedy Decoding Is Not Precision-Invariant", abstract: the top-two margin
    measured against the directional perturbation between the two candidates decides the
    flip).  Steps where B's top two are a different pair carry no d (counted separately).

Random-init weights cannot reproduce the pages' agreement rates (those come from trained
models on benchmark prompts); the harness reproduces the mechanism and measures it on the
library's own kernels.  Every token comes from ``Decoder`` (HIP kernels through the C ABI);
this module only drives the loop and does host bookkeeping.
"""
import numpy as np
import torch

OUT_KEYS = ("tokens", "margin", "top1", "top2", "recomputed")


def greedy(dec, prompts, steps):
    """Greedy continuation of ``prompts`` (device int32 [B, P], P >= 1, B <= dec.batch) for
    ``steps`` tokens: the prompt minus its last token is prefilled, then every step decodes one
    token per sequence and feeds back its top-1.  Returns host arrays [B, steps]: tokens (the
    generated tokens), margin, top1, top2 and recomputed of the LM head at each step."""
    B, P = prompts.shape
    if P < 1 or steps < 1:
        raise ValueError("need a non-empty prompt and at least one step")
    if P + steps - 1 > dec.tmax:
        raise ValueError("prompt + continuation exceed the cache length")
    if P > 1:
        dec.prefill(prompts[:, :P - 1].contiguous())
    tok = prompts[:, P - 1].contiguous()
    tgt = torch.zeros(B, dtype=torch.int32, device=prompts.device)
    rec = {k: [] for k in OUT_KEYS if k != "tokens"}
    toks = []
    for s in range(steps):
        pos = torch.full((B,), P - 1 + s, dtype=torch.int32, device=prompts.device)
        r = dec.decode_step(tok, pos, tgt)
        for k in rec:
            rec[k].append(r[k].clone())
        tok = r["top1"].clone()
        toks.append(tok)
    torch.cuda.synchronize(prompts.device)
    out = {k: torch.stack(v, dim=1).cpu().numpy() for k, v in rec.items()}
    out["tokens"] = torch.stack(toks, dim=1).cpu().numpy()
    return out


def divergence_index(ta, tb):
    """First position where two token rows differ, per row; the row length if they never do."""
    ta, tb = np.asarray(ta), np.asarray(tb)
    diff = ta != tb
    return np.where(diff.any(axis=1), diff.argmax(axis=1), ta.shape[1])


def compare(a, b):
    """Compare two ``greedy`` outputs on the same prompts.  Returns a dict with per-prompt
    divergence indices, exact agreement, and the flip/margin statistics of the steps whose
    prefixes are identical (every step up to and including each prompt's divergence)."""
    ta, tb = a["tokens"], b["tokens"]
    B, S = ta.shape
    di = divergence_index(ta, tb)
    mA, mB = a["margin"].astype(np.float64), b["margin"].astype(np.float64)
    a1, a2, b1, b2 = a["top1"], a["top2"], b["top1"], b["top2"]
    steps = np.arange(S)[None, :]
    comparable = steps <= di[:, None]
    flip = comparable & (a1 != b1)
    same_pair = comparable & (((a1 == b1) & (a2 == b2)) | ((a1 == b2) & (a2 == b1)))
    gB = np.where(a1 == b1, mB, -mB)
    d = np.where(same_pair, mA - gB, np.nan)
    nf = flip & same_pair
    kf = comparable & ~flip & same_pair

    def med(x):
        return float(np.median(x)) if x.size else None

    return {
        "prompts": int(B), "steps": int(S),
        "exact_agreement": float(np.mean(di == S)),
        "divergence_index": di.tolist(),
        "mean_divergence_index": float(np.mean(di)),
        "median_divergence_index_of_diverging": med(di[di < S]),
        "comparable_steps": int(comparable.sum()),
        "flips": int(flip.sum()),
        "flips_other_pair": int((flip & ~same_pair).sum()),
        "median_margin_at_flip": med(mA[nf]),
        "median_margin_no_flip": med(mA[kf]),
        "median_abs_perturbation_at_flip": med(np.abs(d[nf])),
        "median_abs_perturbation_no_flip": med(np.abs(d[kf])),
        # the mechanism: with the same top-two pair, B flips exactly when d > m_A, or when
        # d == m_A (B ties the pair) and the lower index, which wins ties, is a2
        "flip_iff_perturbation_exceeds_margin": bool(np.all(
            ((d > mA) | ((d == mA) & (a2 < a1)))[same_pair] == flip[same_pair])),
        "recompute_rate_a": float(np.mean(a["recomputed"][comparable])),
        "recompute_rate_b": float(np.mean(b["recomputed"][comparable])),
    }


def margin_histogram(a, edges=(0.0, 0.01, 0.03, 0.1, 0.3, 1.0, np.inf)):
    """Counts of run A's per-step margins in the given bins (all steps)."""
    h, _ = np.histogram(np.asarray(a["margin"], np.float64).ravel(), bins=np.asarray(edges))
    return {"edges": [float(e) for e in edges], "counts": h.tolist()}
