"""Float64 brute-force reference of the same mathematics (no fixed order, no rounding to
binary32 inside).  Used only by the tests to pin the oracle: the oracle must agree with
these values within floating-point error bounds.

TEST INFRASTRUCTURE ONLY.

Each function is the textbook definition of the step it names:
  matmul (LayerCast: BF16 weights, computed here in float64)
  RMSNorm, rotate-half RoPE, causal softmax attention, SwiGLU,
  log-softmax / top-2 / logit margin of the LM head
  (the "Greedy Decoding Is Not Precision-Invariant" abstract defines the margin as the
  gap between the two largest logits).
"""
import numpy as np


def up(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm(X, W16):
    return np.asarray(X, np.float64) @ up(W16).T


def rmsnorm(X, gamma16, eps=1e-5):
    X = np.asarray(X, np.float64)
    r = 1.0 / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + float(np.float32(eps)))
    return X * r * up(gamma16)


def rope(X, pos, cos_t, sin_t):
    X = np.asarray(X, np.float64)
    D = X.shape[-1]
    h = D // 2
    c = np.asarray(cos_t, np.float64)[np.asarray(pos)][:, None, :]
    s = np.asarray(sin_t, np.float64)[np.asarray(pos)][:, None, :]
    a, b = X[..., :h], X[..., h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def attention(Q, Kc, Vc, q_start=0, scale=None):
    """Causal softmax attention; Q [B, Tq, Hq, D], caches [B, Hkv, Tmax, D] (fp32 or BF16 bits)."""
    def f(a):
        return up(a) if a.dtype == np.uint16 else np.asarray(a, np.float64)
    Q, Kc, Vc = f(Q), f(Kc), f(Vc)
    B, Tq, Hq, D = Q.shape
    Hkv = Kc.shape[1]
    grp = Hq // Hkv
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    O = np.empty((B, Tq, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            nk = q_start + Tq
            S = (Q[b, :, h, :] @ Kc[b, g, :nk, :].T) * scale
            i = np.arange(Tq)[:, None] + q_start
            j = np.arange(nk)[None, :]
            S = np.where(j <= i, S, -np.inf)
            S = S - S.max(axis=1, keepdims=True)
            P = np.exp(S)
            P = P / P.sum(axis=1, keepdims=True)
            O[b, :, h, :] = P @ Vc[b, g, :nk, :]
    return O


def swiglu(G, U):
    G = np.asarray(G, np.float64)
    return G / (1.0 + np.exp(-G)) * np.asarray(U, np.float64)


def lmhead_pass(A, W16, target):
    """log-softmax at the target, top-2 indices (lowest index on ties) and margin, in float64.
    A is the activation the pass uses (already rounded to BF16 for the P pass)."""
    Z = np.asarray(A, np.float64) @ up(W16).T
    B, V = Z.shape
    M = Z.max(axis=1, keepdims=True)
    lse = M[:, 0] + np.log(np.exp(Z - M).sum(axis=1))
    lp = Z[np.arange(B), target] - lse
    order = np.lexsort((np.broadcast_to(np.arange(V), Z.shape), -Z), axis=1)
    t1 = order[:, 0]
    t2 = order[:, 1]
    margin = Z[np.arange(B), t1] - Z[np.arange(B), t2]
    return dict(logprob=lp, margin=margin, top1=t1, top2=t2, logits=Z)


def store(x, fmt):
    """Storage rounding of an activation: "fp32" keeps the float64 value, "fp16" rounds it to
    the nearest binary16 (NumPy's conversion), "bf16" to the nearest bfloat16 (through the
    nearest binary32, then the top 16 bits with ties to even)."""
    x = np.asarray(x, np.float64)
    if fmt == "fp16":
        return x.astype(np.float16).astype(np.float64)
    if fmt == "bf16":
        u = x.astype(np.float32).view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x


def decoder(tokens, model, eps=1e-5, act="fp32"):
    """Float64 forward of the same decoder; returns the final normed hidden [T, H].  With
    ``act`` "bf16" or "fp16" every activation an unfused implementation stores between
    operations (embedding, norm outputs, projection outputs, rotated q and k, attention
    output, the SwiGLU product, residual sums) is rounded to that format."""
    cfg = model["cfg"]
    H, Hq, Hkv, D, F = (cfg[k] for k in ("hidden", "hq", "hkv", "d", "ffn"))
    T = len(tokens)
    R = lambda a: store(a, act)  # noqa: E731
    x = R(up(model["emb"])[np.asarray(tokens)])
    pos = np.arange(T)
    for layer in model["layers"]:
        n = R(rmsnorm(x, layer["g1"], eps))
        qkv = R(gemm(n, layer["wqkv"]))
        q = R(rope(qkv[:, :Hq * D].reshape(T, Hq, D), pos, model["cos"], model["sin"]))
        k = R(rope(qkv[:, Hq * D:(Hq + Hkv) * D].reshape(T, Hkv, D), pos, model["cos"], model["sin"]))
        v = qkv[:, (Hq + Hkv) * D:].reshape(T, Hkv, D)
        att = R(attention(q[None], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None])[0])
        x = R(x + R(gemm(att.reshape(T, Hq * D), layer["wo"])))
        n = R(rmsnorm(x, layer["g2"], eps))
        gu = R(gemm(n, layer["w13"]))
        x = R(x + R(gemm(R(swiglu(gu[:, :F], gu[:, F:])), layer["w2"])))
    return R(rmsnorm(x, model["gf"], eps))
