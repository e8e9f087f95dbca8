"""ctypes wrapper around the CPU oracle (liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke()`` and by
the benchmark's cpu_baseline leg.  The product path never imports this module.

Every function takes and returns NumPy arrays.  BF16 tensors are carried as ``uint16``
bit patterns, FP32 tensors as ``float32``.  See ``oracle.c`` for the order of every
operation; this file only marshals arguments.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None

f32p = ctypes.POINTER(ctypes.c_float)
u16p = ctypes.POINTER(ctypes.c_uint16)
i32p = ctypes.POINTER(ctypes.c_int32)
u8p = ctypes.POINTER(ctypes.c_uint8)
i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from oracle import build as _b  # noqa: WPS433 (build on first use)
            _b.build()
        L = ctypes.CDLL(LIB_PATH)
        L.orc_exp_f.restype = ctypes.c_float
        L.orc_exp_f.argtypes = [ctypes.c_float]
        L.orc_log_f.restype = ctypes.c_float
        L.orc_log_f.argtypes = [ctypes.c_float]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_add_f32.restype = ctypes.c_float
        L.orc_add_f32.argtypes = [ctypes.c_float, ctypes.c_float]
        L.orc_add_bf16.restype = ctypes.c_uint16
        L.orc_add_bf16.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.orc_dot_ks.restype = ctypes.c_float
        L.orc_dot_ks.argtypes = [f32p, f32p, i64]
        L.orc_constants.restype = ctypes.c_int
        L.orc_constants.argtypes = [f32p, ctypes.c_int]
        L.orc_int_constants.restype = ctypes.c_int
        L.orc_int_constants.argtypes = [i32p, ctypes.c_int]
        L.orc_exp_f_array.argtypes = [f32p, f32p, i64]
        L.orc_log_f_array.argtypes = [f32p, f32p, i64]
        L.orc_bf16_rne_array.argtypes = [f32p, u16p, i64]
        L.orc_f16_rne.restype = ctypes.c_uint16
        L.orc_f16_rne.argtypes = [ctypes.c_float]
        L.orc_f16_up.restype = ctypes.c_float
        L.orc_f16_up.argtypes = [ctypes.c_uint16]
        L.orc_round_act_array.argtypes = [f32p, i64, ctypes.c_int, f32p]
        L.orc_lmhead_logit_grad.argtypes = [f32p, i64, i64, i64, u16p, i64, i32p, f32p, f32p, i64, f32p]
        L.orc_gemm_backward.argtypes = [f32p, i64, i64, i64, f32p, i64, i64, u16p, i64,
                                        f32p, i64, f32p, i64]
        L.orc_gemm_backward_at.argtypes = [ctypes.c_int, f32p, i64, i64, i64, f32p, i64, i64, u16p, i64,
                                           ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                           i64, f32p]
        L.orc_gemm.argtypes = [f32p, i64, i64, i64, u16p, i64, i64, f32p, i64]
        L.orc_rmsnorm.argtypes = [f32p, i64, i64, i64, u16p, ctypes.c_float, f32p, i64]
        L.orc_rope.argtypes = [f32p, i64, i64, i64, i64, i32p, f32p, f32p, f32p, i64]
        L.orc_attention.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    i64, i64, i64, i64, i64, i64, i64, ctypes.c_float, f32p]
        L.orc_swiglu.argtypes = [f32p, f32p, i64, i64, i64, i64, f32p, i64]
        L.orc_set_threads.restype = ctypes.c_int
        L.orc_set_threads.argtypes = [ctypes.c_int]
        L.orc_lmhead_stats.argtypes = [f32p, i64, f32p, f32p, i32p, i32p]
        L.orc_lmhead.argtypes = [f32p, i64, i64, i64, u16p, i64, i32p, ctypes.c_float, ctypes.c_int,
                                 f32p, f32p, i32p, i32p, u8p]
        L.orc_decoder.argtypes = [i32p, i64, i64, i64, i64, i64, i64, i64, i64,
                                  u16p, ctypes.POINTER(u16p), u16p, u16p, f32p, f32p,
                                  ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int, i32p,
                                  f32p, f32p, i32p, i32p, u8p, f32p]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a, ptype):
    return a.ctypes.data_as(ptype)


# ---------------------------------------------------------------- scalars --

def exp_f(x):
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().orc_exp_f_array(_p(x, f32p), _p(y, f32p), x.size)
    return y


def log_f(x):
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().orc_log_f_array(_p(x, f32p), _p(y, f32p), x.size)
    return y


def bf16_rne(x):
    x = _c(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    lib().orc_bf16_rne_array(_p(x, f32p), _p(y, u16p), x.size)
    return y


def bf16_up(b):
    """BF16 bits -> FP32 (the 16 bits become the top half of the word)."""
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# activation storage formats of the decoder: FP32 (LayerCast), BF16, FP16
ACT_FORMATS = {"fp32": 0, "bf16": 1, "fp16": 2}


def round_act(x, fmt):
    """Round FP32 values to the storage format ``fmt`` ("fp32", "bf16", "fp16") and widen the
    result back to FP32."""
    x = _c(x, np.float32)
    y = np.empty_like(x)
    lib().orc_round_act_array(_p(x, f32p), x.size, ACT_FORMATS[fmt], _p(y, f32p))
    return y


def add_f32(a, b):
    return np.float32(lib().orc_add_f32(float(a), float(b)))


def add_bf16(a_bits, b_bits):
    return int(lib().orc_add_bf16(int(a_bits), int(b_bits)))


def dot_ks(x, w):
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    assert x.shape == w.shape and x.ndim == 1
    return np.float32(lib().orc_dot_ks(_p(x, f32p), _p(w, f32p), x.size))


def set_threads(n):
    """Threads of the oracle's parallel loops (independent outputs only); 0 = default.
    Returns the count now in effect."""
    return int(lib().orc_set_threads(int(n)))


def constants():
    """(float constants, int constants) in the oracle's fixed order."""
    f = np.zeros(64, np.float32)
    n = lib().orc_constants(_p(f, f32p), 64)
    i = np.zeros(16, np.int32)
    m = lib().orc_int_constants(_p(i, i32p), 16)
    return f[:n].copy(), i[:m].copy()


# ---------------------------------------------------------------- kernels --

def gemm(X, W):
    """Y = dot_KS(X[m], up(W[n])) for all m, n.  X fp32 [M, K], W bf16 bits [N, K]."""
    X = _c(X, np.float32)
    W = _c(W, np.uint16)
    M, K = X.shape
    N, K2 = W.shape
    assert K == K2
    Y = np.empty((M, N), np.float32)
    lib().orc_gemm(_p(X, f32p), M, K, K, _p(W, u16p), N, K, _p(Y, f32p), N)
    return Y


def lmhead_logit_grad(Hs, W, target, coef):
    """Gradient of coef[b] * lp_b with respect to the FP32-pass logits: G [B, V] with
    G[b, v] = coef[b] * ([v == target_b] - exp_f(z_v - M) / S); also returns lp [B]."""
    Hs = _c(Hs, np.float32)
    W = _c(W, np.uint16)
    target = _c(target, np.int32)
    coef = _c(coef, np.float32)
    B, K = Hs.shape
    V, K2 = W.shape
    assert K == K2 and target.shape == (B,) and coef.shape == (B,)
    G = np.empty((B, V), np.float32)
    lp = np.empty(B, np.float32)
    lib().orc_lmhead_logit_grad(_p(Hs, f32p), B, K, K, _p(W, u16p), V, _p(target, i32p), _p(coef, f32p),
                                _p(G, f32p), V, _p(lp, f32p))
    return G, lp


def gemm_backward(dY, X, W, dx=True, dw=True):
    """Backward of Y = X up(W)^T: dX = dY up(W) (sum over the N outputs) and dW = dY^T X
    (sum over the M tokens), each in the dot_KS order along the reduced index.
    dY fp32 [M, N], X fp32 [M, K], W bf16 bits [N, K].  Returns (dX or None, dW or None)."""
    dY = _c(dY, np.float32)
    X = _c(X, np.float32)
    W = _c(W, np.uint16)
    M, N = dY.shape
    M2, K = X.shape
    assert M == M2 and W.shape == (N, K)
    gx = np.empty((M, K), np.float32) if dx else None
    gw = np.empty((N, K), np.float32) if dw else None
    lib().orc_gemm_backward(_p(dY, f32p), M, N, N, _p(X, f32p), K, K, _p(W, u16p), K,
                            _p(gx, f32p) if dx else None, K, _p(gw, f32p) if dw else None, K)
    return gx, gw


def gemm_backward_at(which, dY, X, W, rows, cols):
    """Single outputs of the same definitions: dX[rows[i], cols[i]] (which "dx") or
    dW[rows[i], cols[i]] (which "dw")."""
    dY = _c(dY, np.float32)
    X = _c(X, np.float32)
    W = _c(W, np.uint16)
    M, N = dY.shape
    K = X.shape[1]
    rows = _c(rows, np.int64)
    cols = _c(cols, np.int64)
    out = np.empty(rows.shape[0], np.float32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib().orc_gemm_backward_at(0 if which == "dx" else 1, _p(dY, f32p), M, N, N, _p(X, f32p), K, K,
                               _p(W, u16p), K, _p(rows, i64p), _p(cols, i64p), rows.shape[0], _p(out, f32p))
    return out


def rmsnorm(X, gamma, eps=1e-5):
    X = _c(X, np.float32)
    gamma = _c(gamma, np.uint16)
    M, H = X.shape
    Y = np.empty_like(X)
    lib().orc_rmsnorm(_p(X, f32p), M, H, H, _p(gamma, u16p), float(np.float32(eps)), _p(Y, f32p), H)
    return Y


def rope(X, pos, cos_t, sin_t):
    """X fp32 [M, nh, D] at positions pos[M]; tables fp32 [Tmax, D/2]."""
    X = _c(X, np.float32)
    M, nh, D = X.shape
    pos = _c(pos, np.int32)
    cos_t = _c(cos_t, np.float32)
    sin_t = _c(sin_t, np.float32)
    Y = np.empty_like(X)
    lib().orc_rope(_p(X, f32p), M, nh, D, nh * D, _p(pos, i32p), _p(cos_t, f32p), _p(sin_t, f32p),
                   _p(Y, f32p), nh * D)
    return Y


def attention(Q, Kc, Vc, q_start=0, scale=None):
    """Causal attention.  Q [B, Tq, Hq, D]; Kc, Vc [B, Hkv, Tmax, D]; either all BF16 bits
    (uint16) or all fp32.  Returns fp32 [B, Tq, Hq, D]."""
    bf = Q.dtype == np.uint16
    dt = 0 if bf else 1
    typ = np.uint16 if bf else np.float32
    Q = _c(Q, typ)
    Kc = _c(Kc, typ)
    Vc = _c(Vc, typ)
    B, Tq, Hq, D = Q.shape
    B2, Hkv, Tmax, D2 = Kc.shape
    assert B == B2 and D == D2 and Hq % Hkv == 0 and q_start + Tq <= Tmax
    if scale is None:
        scale = np.float32(1.0) / np.sqrt(np.float32(D))
    O = np.empty((B, Tq, Hq, D), np.float32)
    lib().orc_attention(dt, Q.ctypes.data, Kc.ctypes.data, Vc.ctypes.data, B, Tq, q_start, Tmax,
                        Hq, Hkv, D, float(np.float32(scale)), _p(O, f32p))
    return O


def swiglu(G, U):
    G = _c(G, np.float32)
    U = _c(U, np.float32)
    M, F = G.shape
    Hh = np.empty_like(G)
    lib().orc_swiglu(_p(G, f32p), _p(U, f32p), M, F, F, F, _p(Hh, f32p), F)
    return Hh


def lmhead_stats(z):
    """Row statistics of one FP32 logit row: (M, S, top1, top2) with S the fixed tile/lane
    tree of exp_f(z_v - M)."""
    z = _c(z, np.float32)
    assert z.ndim == 1 and z.size >= 2
    M = np.zeros(1, np.float32)
    S = np.zeros(1, np.float32)
    t1 = np.zeros(1, np.int32)
    t2 = np.zeros(1, np.int32)
    lib().orc_lmhead_stats(_p(z, f32p), z.size, _p(M, f32p), _p(S, f32p), _p(t1, i32p), _p(t2, i32p))
    return M[0], S[0], int(t1[0]), int(t2[0])


def lmhead(Hs, W, target, tau=np.float32(0.1), mode=0):
    """Selective-recompute LM head on rows of Hs (fp32 [B, K]) with W bf16 bits [V, K].
    mode 0: selective; 1: P pass only; 2: F pass only."""
    Hs = _c(Hs, np.float32)
    W = _c(W, np.uint16)
    target = _c(target, np.int32)
    B, K = Hs.shape
    V, K2 = W.shape
    assert K == K2 and target.shape == (B,)
    lp = np.empty(B, np.float32)
    mg = np.empty(B, np.float32)
    t1 = np.empty(B, np.int32)
    t2 = np.empty(B, np.int32)
    fl = np.empty(B, np.uint8)
    lib().orc_lmhead(_p(Hs, f32p), B, K, K, _p(W, u16p), V, _p(target, i32p), float(np.float32(tau)), mode,
                     _p(lp, f32p), _p(mg, f32p), _p(t1, i32p), _p(t2, i32p), _p(fl, u8p))
    return dict(logprob=lp, margin=mg, top1=t1, top2=t2, recomputed=fl)


def decoder(tokens, model, eps=1e-5, tau=np.float32(0.1), return_hidden=False, act="fp32",
            targets=None):
    """Score one sequence with the Llama-shaped decoder.  ``model`` is the dict built by
    ``synth.decoder_model`` (BF16 weights as uint16 bits, RoPE tables fp32).  ``act`` is the
    activation storage format.  By default positions 0..T-2 are scored against the next
    token; with ``targets`` (int32 [T]) all T positions are scored against those."""
    cfg = model["cfg"]
    H, Hq, Hkv, D, F, V, L = (cfg[k] for k in ("hidden", "hq", "hkv", "d", "ffn", "vocab", "layers"))
    tokens = _c(tokens, np.int32)
    T = tokens.shape[0]
    keep = []
    ptrs = (u16p * (6 * L))()
    for li, layer in enumerate(model["layers"]):
        for j, name in enumerate(("g1", "wqkv", "wo", "g2", "w13", "w2")):
            a = _c(layer[name], np.uint16)
            keep.append(a)
            ptrs[6 * li + j] = _p(a, u16p)
    emb = _c(model["emb"], np.uint16)
    gf = _c(model["gf"], np.uint16)
    wh = _c(model["whead"], np.uint16)
    cos_t = _c(model["cos"], np.float32)
    sin_t = _c(model["sin"], np.float32)
    assert cos_t.shape[0] >= T
    if targets is None:
        tgt = np.zeros(T, np.int32)
        tgt[:T - 1] = tokens[1:]
        nout = T - 1
    else:
        tgt = _c(targets, np.int32)
        assert tgt.shape == (T,)
        nout = T
    lp = np.empty(T, np.float32)
    mg = np.empty(T, np.float32)
    t1 = np.empty(T, np.int32)
    t2 = np.empty(T, np.int32)
    fl = np.empty(T, np.uint8)
    hid = np.empty((T, H), np.float32) if return_hidden else None
    scale = np.float32(1.0) / np.sqrt(np.float32(D))
    lib().orc_decoder(_p(tokens, i32p), T, H, Hq, Hkv, D, F, V, L, _p(emb, u16p), ptrs, _p(gf, u16p),
                      _p(wh, u16p), _p(cos_t, f32p), _p(sin_t, f32p), float(np.float32(eps)),
                      float(scale), float(np.float32(tau)), ACT_FORMATS[act], _p(tgt, i32p),
                      _p(lp, f32p), _p(mg, f32p), _p(t1, i32p), _p(t2, i32p), _p(fl, u8p),
                      _p(hid, f32p) if hid is not None else None)
    out = dict(logprob=lp[:nout], margin=mg[:nout], top1=t1[:nout], top2=t2[:nout],
               recomputed=fl[:nout])
    if return_hidden:
        out["hidden"] = hid
    return out


def greedy(prompt, model, steps, act="fp32", tau=np.float32(0.1), eps=1e-5):
    """Greedy continuation of one prompt: each new token is the top-1 of the LM head at the
    last position, recomputed from scratch over the whole sequence at every step.  Returns
    int32 tokens [steps] and the per-step LM-head outputs (margin, top1, top2, recomputed)."""
    seq = [int(t) for t in np.asarray(prompt)]
    rec = {k: [] for k in ("margin", "top1", "top2", "recomputed")}
    for _ in range(steps):
        r = decoder(np.asarray(seq, np.int32), model, eps=eps, tau=tau, act=act,
                    targets=np.zeros(len(seq), np.int32))
        for k in rec:
            rec[k].append(r[k][-1])
        seq.append(int(r["top1"][-1]))
    out = {k: np.asarray(v) for k, v in rec.items()}
    out["tokens"] = np.asarray(seq[len(prompt):], np.int32)
    return out
