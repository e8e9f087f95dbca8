"""Thin ctypes binding of libinvnum.so.

Each ``inv_*`` function below has the name of the C entry point it calls and only
marshals arguments: torch tensors supply device pointers, torch's current stream is
passed as the HIP stream, and every step of the computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing the import of this module
fails, and a non-zero status raises ``InvError``.
"""
import ctypes
import os
import struct

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libinvnum.so")

INV_BF16 = 0
INV_F32 = 1

i64 = ctypes.c_int64
vp = ctypes.c_void_p


class InvError(RuntimeError):
    pass


class _Consts(ctypes.Structure):
    _fields_ = [("ks", ctypes.c_int32), ("chunk", ctypes.c_int32), ("vocab_tile", ctypes.c_int32),
                ("lanes", ctypes.c_int32), ("n_float", ctypes.c_int32),
                ("float_consts", ctypes.c_float * 32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libinvnum.so is not built (run __graft_entry__.build() or "
                          "python invariant_numerics_amd/build.py); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "inv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "inv_get_constants": (ctypes.c_int, [ctypes.POINTER(_Consts)]),
        "inv_fixed_order_gemm": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, i64, vp, i64, vp, i64, vp]),
        "inv_rmsnorm": (ctypes.c_int, [vp, i64, i64, i64, vp, ctypes.c_float, vp, i64, vp]),
        "inv_gated_gemm": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, i64, vp, i64, vp]),
        "inv_attention_prefill": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                                 i64, ctypes.c_float, vp, vp]),
        "inv_attention_decode_workspace_bytes": (ctypes.c_size_t, [i64, i64, i64, i64]),
        "inv_attention_decode": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                ctypes.c_float, vp, vp, ctypes.c_size_t, vp]),
        "inv_attention_decode_noalloc_max_bytes": (ctypes.c_size_t, []),
        "inv_attention_decode_noalloc": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                        ctypes.c_float, vp, vp]),
        "inv_lmhead_workspace_bytes": (ctypes.c_size_t, [i64, i64, i64]),
        "inv_lmhead_logprob_top2": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, ctypes.c_float, vp, vp,
                                                   vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "inv_embed": (ctypes.c_int, [vp, i64, vp, i64, i64, vp, i64, vp]),
        "inv_rope_kv_append": (ctypes.c_int, [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, i64, i64, vp,
                                              vp, vp, ctypes.c_int, vp]),
        "inv_swiglu": (ctypes.c_int, [vp, vp, i64, i64, i64, i64, vp, i64, vp]),
        "inv_add": (ctypes.c_int, [vp, vp, i64, i64, i64, i64, vp, i64, vp]),
        "inv_round_activations": (ctypes.c_int, [vp, i64, i64, i64, ctypes.c_int, vp, i64, vp]),
        "inv_lmhead_logit_grad_workspace_bytes": (ctypes.c_size_t, [i64, i64, i64]),
        "inv_lmhead_logit_grad": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                                 vp]),
        "inv_gemm_backward_workspace_bytes": (ctypes.c_size_t, [i64, i64, i64]),
        "inv_gemm_backward": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, i64, vp, i64, vp, i64, vp, i64,
                                             vp, ctypes.c_size_t, vp]),
        "inv_eval_numerics": (ctypes.c_int, [ctypes.c_int, vp, vp, i64, vp]),
        "inv_mfma_f32_check": (ctypes.c_int, [vp, vp, vp, vp, i64, vp]),
        "inv_mfma32_f32_check": (ctypes.c_int, [vp, vp, vp, vp, i64, vp]),
        "inv_mfma_bf16_check": (ctypes.c_int, [vp, vp, vp, vp, i64, vp]),
        "inv_qkv_rope_kv_append_workspace_bytes": (ctypes.c_size_t, [i64, i64, i64, i64]),
        "inv_qkv_rope_kv_append": (ctypes.c_int, [vp, i64, i64, i64, vp, i64, i64, i64, i64, vp, vp, vp, vp, i64,
                                                  i64, vp, vp, vp, vp, ctypes.c_size_t, vp]),
        "inv_read_stream_probe": (ctypes.c_int, [vp, i64, vp, i64, vp]),
        "inv_mfma_rate_probe": (ctypes.c_int, [ctypes.c_int, i64, i64, vp, vp]),
        "inv_attention_prefill_workspace_bytes": (ctypes.c_size_t, [i64, i64, i64, i64, i64]),
        "inv_attention_prefill_ws": (ctypes.c_int, [ctypes.c_int, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64,
                                                    ctypes.c_float, vp, vp, ctypes.c_size_t, vp]),
        "inv_kernel_route": (ctypes.c_int, [ctypes.c_int, i64, i64, ctypes.c_char_p, ctypes.c_size_t]),
        "inv_rmsnorm_gemm": (ctypes.c_int, [vp, i64, i64, i64, vp, ctypes.c_float, vp, i64, i64, vp, i64, vp, i64,
                                            ctypes.c_int, vp]),
        "inv_rmsnorm_qkv_rope_kv_append": (ctypes.c_int, [vp, i64, i64, i64, vp, ctypes.c_float, vp, i64, i64, i64,
                                                          i64, vp, vp, vp, vp, i64, i64, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


LIB = _load()
EXPORTS = ("inv_status_string", "inv_get_constants", "inv_fixed_order_gemm", "inv_gated_gemm", "inv_rmsnorm",
           "inv_attention_prefill", "inv_attention_decode_workspace_bytes", "inv_attention_decode",
           "inv_lmhead_workspace_bytes", "inv_lmhead_logprob_top2", "inv_embed", "inv_rope_kv_append",
           "inv_swiglu", "inv_add", "inv_round_activations", "inv_lmhead_logit_grad_workspace_bytes",
           "inv_lmhead_logit_grad", "inv_gemm_backward_workspace_bytes",
           "inv_gemm_backward", "inv_eval_numerics", "inv_mfma_f32_check", "inv_mfma32_f32_check",
           "inv_mfma_bf16_check", "inv_kernel_route", "inv_attention_decode_noalloc",
           "inv_attention_decode_noalloc_max_bytes", "inv_qkv_rope_kv_append_workspace_bytes",
           "inv_qkv_rope_kv_append", "inv_read_stream_probe", "inv_mfma_rate_probe",
           "inv_attention_prefill_workspace_bytes", "inv_attention_prefill_ws", "inv_rmsnorm_gemm",
           "inv_rmsnorm_qkv_rope_kv_append")


def _check(status, what):
    if status != 0:
        raise InvError("%s: %s (%d)" % (what, LIB.inv_status_string(status).decode(), status))


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _p(t):
    return None if t is None else t.data_ptr()


def _dev(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise InvError("tensors must be on the GPU (the library runs HIP kernels only)")


def _bf16(t):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise InvError("BF16 operand expected (bfloat16 or its 16-bit pattern), got %s" % t.dtype)
    return t


def _f32(t):
    if t.dtype != torch.float32:
        raise InvError("float32 operand expected, got %s" % t.dtype)
    return t


def _row_ld(t):
    if t.dim() != 2 or t.stride(1) != 1:
        raise InvError("2-D row-major tensor with unit inner stride expected")
    return t.stride(0)


# --------------------------------------------------------------------------- host --

def inv_status_string(status):
    return LIB.inv_status_string(int(status)).decode()


def inv_get_constants():
    c = _Consts()
    _check(LIB.inv_get_constants(ctypes.byref(c)), "inv_get_constants")
    return dict(ks=c.ks, chunk=c.chunk, vocab_tile=c.vocab_tile, lanes=c.lanes,
                float_consts=[c.float_consts[i] for i in range(c.n_float)])


ROUTE_OPS = {"gemm": 0, "gated_gemm": 1, "lmhead_gemm": 2, "attention_prefill": 3}


def inv_kernel_route(op, a, b):
    """Name of the kernel instantiation a call launches (host-only query): op "gemm" (a = M,
    b = N), "gated_gemm" (a = M, b = N2), "lmhead_gemm" (a = B, b = V, tau > 0) or
    "attention_prefill" (a = B * Hq, b = Tq)."""
    if op not in ROUTE_OPS:
        raise InvError("unknown route op %r" % (op,))
    buf = ctypes.create_string_buffer(128)
    _check(LIB.inv_kernel_route(ROUTE_OPS[op], int(a), int(b), buf, len(buf)), "inv_kernel_route")
    return buf.value.decode()


def inv_attention_decode_workspace_bytes(B, Tmax, Hq, D):
    return int(LIB.inv_attention_decode_workspace_bytes(B, Tmax, Hq, D))


def inv_lmhead_workspace_bytes(B, K, V):
    return int(LIB.inv_lmhead_workspace_bytes(B, K, V))


# ------------------------------------------------------------------------- device --

def inv_fixed_order_gemm(X, W, R=None, out=None):
    """Y = X . up(W)^T (+ R), X fp32 [M, K], W bf16 [N, K]."""
    _dev(X, W, R, out)
    _f32(X)
    _bf16(W)
    M, K = X.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=X.device)
    _check(LIB.inv_fixed_order_gemm(_p(X), M, K, _row_ld(X), _p(W), N, _row_ld(W), _p(R),
                                    _row_ld(R) if R is not None else 0, _p(out), _row_ld(out),
                                    _stream(X)), "inv_fixed_order_gemm")
    return out


def inv_gated_gemm(X, W, out=None):
    """H = silu(X . up(W[0::2])^T) * (X . up(W[1::2])^T): W bf16 [N2, K] with gate/up rows
    interleaved; H fp32 [M, N2/2]."""
    _dev(X, W, out)
    _f32(X)
    _bf16(W)
    M, K = X.shape
    N2 = W.shape[0]
    if out is None:
        out = torch.empty((M, N2 // 2), dtype=torch.float32, device=X.device)
    _check(LIB.inv_gated_gemm(_p(X), M, K, _row_ld(X), _p(W), N2, _row_ld(W), _p(out), _row_ld(out),
                              _stream(X)), "inv_gated_gemm")
    return out


def inv_rmsnorm(X, gamma, eps=1e-5, out=None):
    _dev(X, gamma, out)
    _f32(X)
    _bf16(gamma)
    M, H = X.shape
    if out is None:
        out = torch.empty_like(X)
    _check(LIB.inv_rmsnorm(_p(X), M, H, _row_ld(X), _p(gamma), float(eps), _p(out), _row_ld(out),
                           _stream(X)), "inv_rmsnorm")
    return out


def inv_rmsnorm_gemm(X, gamma, W, eps=1e-5, R=None, out=None, gated=False):
    """inv_rmsnorm(X, gamma, eps) then inv_fixed_order_gemm (or inv_gated_gemm when gated) on
    the normalised rows, in one launch; X fp32 [M, K] with M <= 4, gamma bf16 [K]."""
    _dev(X, gamma, W, R, out)
    _f32(X)
    _bf16(gamma)
    _bf16(W)
    M, K = X.shape
    N = W.shape[0]
    if out is None:
        out = torch.empty((M, N // 2 if gated else N), dtype=torch.float32, device=X.device)
    _check(LIB.inv_rmsnorm_gemm(_p(X), M, K, _row_ld(X), _p(gamma), float(eps), _p(W), N, _row_ld(W), _p(R),
                                0 if R is None else _row_ld(R), _p(out), _row_ld(out), 1 if gated else 0,
                                _stream(X)), "inv_rmsnorm_gemm")
    return out


def inv_rmsnorm_qkv_rope_kv_append(X, gamma, Wqkv, Hq, Hkv, D, seq, pos, cos_t, sin_t, Qout, Kc, Vc, eps=1e-5):
    """inv_rmsnorm(X, gamma, eps) then inv_qkv_rope_kv_append on the normalised rows, in one
    launch (one to four rows, D = 128)."""
    _dev(X, gamma, Wqkv, seq, pos, cos_t, sin_t, Qout, Kc, Vc)
    _f32(X)
    _bf16(gamma)
    _bf16(Wqkv)
    M, K = X.shape
    Bc, _, Tmax, _ = Kc.shape
    _check(LIB.inv_rmsnorm_qkv_rope_kv_append(_p(X), M, K, _row_ld(X), _p(gamma), float(eps), _p(Wqkv),
                                              _row_ld(Wqkv), Hq, Hkv, D, _p(seq), _p(pos), _p(cos_t), _p(sin_t),
                                              Tmax, Bc, _p(Qout), _p(Kc), _p(Vc), _stream(X)),
           "inv_rmsnorm_qkv_rope_kv_append")
    return Qout


def _ws(need, ws, dev):
    if need == 0:
        return None
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    return ws


def inv_qkv_rope_kv_append(X, Wqkv, Hq, Hkv, D, seq, pos, cos_t, sin_t, Qout, Kc, Vc, ws=None):
    """QKV projection of X (fp32 [M, K]) with RoPE and the KV append (FP32): Qout [M, Hq, D]
    and the caches [Bcache, Hkv, Tmax, D] are written; one launch for up to four rows."""
    _dev(X, Wqkv, seq, pos, cos_t, sin_t, Qout, Kc, Vc, ws)
    _f32(X)
    _bf16(Wqkv)
    M, K = X.shape
    Bc, _, Tmax, _ = Kc.shape
    need = int(LIB.inv_qkv_rope_kv_append_workspace_bytes(M, Hq, Hkv, D))
    ws = _ws(need, ws, X.device)
    _check(LIB.inv_qkv_rope_kv_append(_p(X), M, K, _row_ld(X), _p(Wqkv), _row_ld(Wqkv), Hq, Hkv, D, _p(seq), _p(pos),
                                      _p(cos_t), _p(sin_t), Tmax, Bc, _p(Qout), _p(Kc), _p(Vc), _p(ws),
                                      0 if ws is None else ws.numel() * ws.element_size(), _stream(X)),
           "inv_qkv_rope_kv_append")
    return Qout


def _dtype_code(t):
    if t.dtype == torch.float32:
        return INV_F32
    _bf16(t)
    return INV_BF16


# the pinned attention scale RN(1 / sqrt(128)) (head dim 128, the only one the library runs)
SCALE_D128 = struct.unpack("<f", struct.pack("<I", 0x3DB504F3))[0]


def _scale(D, scale):
    if scale is None:
        if D != 128:
            raise InvError("head dim 128 expected (pass scale explicitly otherwise)")
        scale = SCALE_D128
    return float(scale)


def inv_attention_prefill_workspace_bytes(B, Tq, q_start, Hq, D):
    return int(LIB.inv_attention_prefill_workspace_bytes(B, Tq, q_start, Hq, D))


def inv_attention_prefill(Q, Kc, Vc, q_start=0, scale=None, out=None, split=True, ws=None):
    """Q [B, Tq, Hq, D]; Kc, Vc [B, Hkv, Tmax, D]; returns fp32 [B, Tq, Hq, D].  split: use the
    workspace form (inv_attention_prefill_ws) when the shape has a split path; the same bits."""
    _dev(Q, Kc, Vc, out, ws)
    B, Tq, Hq, D = Q.shape
    _, Hkv, Tmax, _ = Kc.shape
    for t in (Q, Kc, Vc):
        if not t.is_contiguous():
            raise InvError("contiguous tensors expected")
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=torch.float32, device=Q.device)
    need = inv_attention_prefill_workspace_bytes(B, Tq, q_start, Hq, D) if split else 0
    if need:
        ws = _ws(need, ws, Q.device)
        _check(LIB.inv_attention_prefill_ws(_dtype_code(Q), _p(Q), _p(Kc), _p(Vc), B, Tq, q_start, Tmax, Hq, Hkv,
                                            D, _scale(D, scale), _p(out), _p(ws), ws.numel() * ws.element_size(),
                                            _stream(Q)), "inv_attention_prefill_ws")
        return out
    _check(LIB.inv_attention_prefill(_dtype_code(Q), _p(Q), _p(Kc), _p(Vc), B, Tq, q_start, Tmax, Hq, Hkv,
                                     D, _scale(D, scale), _p(out), _stream(Q)), "inv_attention_prefill")
    return out


def inv_attention_decode(Q, Kc, Vc, pos, scale=None, out=None, ws=None):
    """Q [B, Hq, D]; caches [B, Hkv, Tmax, D]; pos int32 [B] (device)."""
    _dev(Q, Kc, Vc, pos, out, ws)
    B, Hq, D = Q.shape
    _, Hkv, Tmax, _ = Kc.shape
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=Q.device)
    need = inv_attention_decode_workspace_bytes(B, Tmax, Hq, D)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=Q.device)
    _check(LIB.inv_attention_decode(_dtype_code(Q), _p(Q), _p(Kc), _p(Vc), _p(pos), B, Tmax, Hq, Hkv, D,
                                    _scale(D, scale), _p(out), _p(ws), ws.numel() * ws.element_size(),
                                    _stream(Q)), "inv_attention_decode")
    return out


def inv_attention_decode_noalloc_max_bytes():
    return int(LIB.inv_attention_decode_noalloc_max_bytes())


def inv_attention_decode_noalloc(Q, Kc, Vc, pos, out, scale=None):
    """inv_attention_decode without a workspace (the library's own per-GPU array holds the
    chunk partials, up to inv_attention_decode_noalloc_max_bytes()); ``out`` [B, Hq, D] FP32 is
    required, so nothing is allocated here either.  Calls that overlap on one GPU race."""
    _dev(Q, Kc, Vc, pos, out)
    B, Hq, D = Q.shape
    _, Hkv, Tmax, _ = Kc.shape
    _check(LIB.inv_attention_decode_noalloc(_dtype_code(Q), _p(Q), _p(Kc), _p(Vc), _p(pos), B, Tmax, Hq, Hkv, D,
                                            _scale(D, scale), _p(out), _stream(Q)), "inv_attention_decode_noalloc")
    return out


def inv_lmhead_logprob_top2(Hs, W, target, tau=0.1, ws=None, out=None):
    """Selective-recompute LM head.  Returns dict of device tensors
    (logprob, margin, top1, top2, recomputed)."""
    _dev(Hs, W, target, ws)
    _f32(Hs)
    _bf16(W)
    B, K = Hs.shape
    V = W.shape[0]
    dev = Hs.device
    if out is None:
        out = dict(logprob=torch.empty(B, dtype=torch.float32, device=dev),
                   margin=torch.empty(B, dtype=torch.float32, device=dev),
                   top1=torch.empty(B, dtype=torch.int32, device=dev),
                   top2=torch.empty(B, dtype=torch.int32, device=dev),
                   recomputed=torch.empty(B, dtype=torch.uint8, device=dev))
    need = inv_lmhead_workspace_bytes(B, K, V)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
    _check(LIB.inv_lmhead_logprob_top2(_p(Hs), B, K, _row_ld(Hs), _p(W), V, _p(target), float(tau),
                                       _p(out["logprob"]), _p(out["margin"]), _p(out["top1"]),
                                       _p(out["top2"]), _p(out["recomputed"]), _p(ws),
                                       ws.numel() * ws.element_size(), _stream(Hs)),
           "inv_lmhead_logprob_top2")
    return out


def inv_embed(ids, table, out=None):
    _dev(ids, table, out)
    M = ids.numel()
    V, H = table.shape
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=ids.device)
    _check(LIB.inv_embed(_p(ids), M, _p(table), V, H, _p(out), _row_ld(out), _stream(ids)), "inv_embed")
    return out


def inv_rope_kv_append(QKV, Hq, Hkv, D, seq, pos, cos_t, sin_t, Qout, Kc, Vc, fmt="fp32"):
    _dev(QKV, seq, pos, cos_t, sin_t, Qout, Kc, Vc)
    if fmt not in ACT_FORMATS:
        raise InvError("unknown activation format %r" % (fmt,))
    M = QKV.shape[0]
    Bc, _, Tmax, _ = Kc.shape
    _check(LIB.inv_rope_kv_append(_p(QKV), M, _row_ld(QKV), Hq, Hkv, D, _p(seq), _p(pos), _p(cos_t),
                                  _p(sin_t), Tmax, Bc, _p(Qout), _p(Kc), _p(Vc), ACT_FORMATS[fmt],
                                  _stream(QKV)),
           "inv_rope_kv_append")
    return Qout


def inv_swiglu(G, U, out=None):
    _dev(G, U, out)
    M, F = G.shape
    if out is None:
        out = torch.empty((M, F), dtype=torch.float32, device=G.device)
    _check(LIB.inv_swiglu(_p(G), _p(U), M, F, _row_ld(G), _row_ld(U), _p(out), _row_ld(out), _stream(G)),
           "inv_swiglu")
    return out


def inv_add(A, Bm, out=None):
    _dev(A, Bm, out)
    M, N = A.shape
    if out is None:
        out = torch.empty_like(A)
    _check(LIB.inv_add(_p(A), _p(Bm), M, N, _row_ld(A), _row_ld(Bm), _p(out), _row_ld(out), _stream(A)),
           "inv_add")
    return out


def inv_lmhead_logit_grad_workspace_bytes(B, K, V):
    return int(LIB.inv_lmhead_logit_grad_workspace_bytes(B, K, V))


def inv_lmhead_logit_grad(Hs, W, target, coef, out=None, logprob=False, ws=None):
    """Gradient of coef[b] * logprob_b (FP32 head) with respect to the logits: FP32 [B, V].
    With logprob=True also returns the FP32-pass logprobs [B]."""
    _dev(Hs, W, target, coef, out, ws)
    B, K = Hs.shape
    V = W.shape[0]
    if out is None:
        out = torch.empty((B, V), dtype=torch.float32, device=Hs.device)
    if out.shape != (B, V) or not out.is_contiguous():
        raise InvError("gradient output must be a contiguous [B, V] FP32 tensor")
    lp = torch.empty(B, dtype=torch.float32, device=Hs.device) if logprob else None
    if ws is None:
        ws = torch.empty(max(1, inv_lmhead_logit_grad_workspace_bytes(B, K, V)), dtype=torch.uint8, device=Hs.device)
    _check(LIB.inv_lmhead_logit_grad(_p(Hs), B, K, _row_ld(Hs), _p(W), V, _p(target), _p(coef), _p(out), _p(lp),
                                     _p(ws), ws.numel(), _stream(Hs)), "inv_lmhead_logit_grad")
    return (out, lp) if logprob else out


def inv_gemm_backward_workspace_bytes(M, N, K):
    return int(LIB.inv_gemm_backward_workspace_bytes(M, N, K))


def inv_gemm_backward(dY, X, W, dx=True, dw=True, out_dx=None, out_dw=None, ws=None):
    """Gradients of Y = inv_fixed_order_gemm(X, W) for the output gradient dY (FP32 [M, N]):
    dX = dY up(W) (FP32 [M, K]) and dW = dY^T X (FP32 [N, K]), each summed in the fixed
    order along its reduced index.  Returns (dX or None, dW or None)."""
    _dev(dY, X, W, out_dx, out_dw, ws)
    M, N = dY.shape
    Nw, K = W.shape
    if Nw != N or (X is not None and tuple(X.shape) != (M, K)):
        raise InvError("shapes: dY [M, N], X [M, K], W [N, K]")
    if dx and out_dx is None:
        out_dx = torch.empty((M, K), dtype=torch.float32, device=dY.device)
    if dw and out_dw is None:
        out_dw = torch.empty((N, K), dtype=torch.float32, device=dY.device)
    if dx and ws is None:
        ws = torch.empty(max(1, inv_gemm_backward_workspace_bytes(M, N, K)), dtype=torch.uint8, device=dY.device)
    _check(LIB.inv_gemm_backward(_p(dY), M, N, _row_ld(dY), _p(X) if dw else None, K,
                                 _row_ld(X) if dw else K, _p(W), _row_ld(W),
                                 _p(out_dx) if dx else None, _row_ld(out_dx) if dx else K,
                                 _p(out_dw) if dw else None, _row_ld(out_dw) if dw else K,
                                 _p(ws) if dx else None, ws.numel() if dx else 0, _stream(dY)),
           "inv_gemm_backward")
    return (out_dx if dx else None), (out_dw if dw else None)


# activation storage formats: name -> dtype code of the C ABI
ACT_FORMATS = {"bf16": 0, "fp32": 1, "fp16": 2}


def inv_round_activations(X, fmt, out=None):
    """Round the FP32 2-D tensor X (unit inner stride) to ``fmt`` ("bf16", "fp16", "fp32")
    and store the widened values in ``out`` (default: a new tensor; ``out=X`` rounds in
    place)."""
    _dev(X, out)
    if X.dtype != torch.float32:
        raise InvError("FP32 activations expected")
    if fmt not in ACT_FORMATS:
        raise InvError("unknown activation format %r" % (fmt,))
    if out is None:
        out = torch.empty(X.shape, dtype=torch.float32, device=X.device)
    rows, cols = X.shape
    _check(LIB.inv_round_activations(_p(X), rows, cols, _row_ld(X), ACT_FORMATS[fmt], _p(out), _row_ld(out),
                                     _stream(X)), "inv_round_activations")
    return out


def inv_eval_numerics(fn, x, out=None):
    _dev(x, out)
    if out is None:
        out = torch.empty_like(x)
    _check(LIB.inv_eval_numerics(int(fn), _p(x), _p(out), x.numel(), _stream(x)), "inv_eval_numerics")
    return out


def inv_mfma_f32_check(A, B, C, out=None):
    """A [n, 16, 4], B [n, 4, 16], C [n, 16, 16] fp32 -> D = C + A B per test, as the
    FP32 matrix instruction computes it."""
    _dev(A, B, C, out)
    n = A.shape[0]
    if out is None:
        out = torch.empty_like(C)
    _check(LIB.inv_mfma_f32_check(_p(A), _p(B), _p(C), _p(out), n, _stream(A)), "inv_mfma_f32_check")
    return out


def inv_mfma32_f32_check(A, B, C, out=None):
    """A [n, 32, 2], B [n, 2, 32], C [n, 32, 32] fp32 -> D = C + A B per test, as the
    32x32x2 FP32 matrix instruction computes it."""
    _dev(A, B, C, out)
    n = A.shape[0]
    if out is None:
        out = torch.empty_like(C)
    _check(LIB.inv_mfma32_f32_check(_p(A), _p(B), _p(C), _p(out), n, _stream(A)), "inv_mfma32_f32_check")
    return out


def inv_mfma_bf16_check(A, B, C, out=None):
    """Lane form of one v_mfma_f32_16x16x32_bf16 per test: A, B [n, 64, 8] BF16 (bits), C
    [n, 64, 4] FP32 -> D [n, 64, 4], each lane's registers as the instruction leaves them."""
    _dev(A, B, C, out)
    n = A.shape[0]
    if tuple(A.shape) != (n, 64, 8) or tuple(B.shape) != (n, 64, 8) or tuple(C.shape) != (n, 64, 4):
        raise InvError("shapes: A, B [n, 64, 8] (BF16), C [n, 64, 4] (FP32)")
    _bf16(A)
    _bf16(B)
    _f32(C)
    if out is None:
        out = torch.empty_like(C)
    _check(LIB.inv_mfma_bf16_check(_p(A), _p(B), _p(C), _p(out), n, _stream(A)), "inv_mfma_bf16_check")
    return out


def inv_read_stream_probe(src, grid=4096, sink=None):
    """Read every byte of the device tensor ``src`` once (diagnostic stream); returns the
    per-workgroup checksums [grid] (uint32 stored as int32)."""
    _dev(src, sink)
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(grid, dtype=torch.int32, device=src.device)
    _check(LIB.inv_read_stream_probe(_p(src), nbytes - nbytes % 16, _p(sink), grid, _stream(src)),
           "inv_read_stream_probe")
    return sink


def inv_mfma_rate_probe(shape, iters, waves_per_cu, out=None, device="cuda"):
    """Back-to-back FP32 matrix instructions (shape 0: 16x16x4, 1: 32x32x2) at waves_per_cu
    wavefronts per CU; returns the output buffer (flops: grid * 4 * iters * 8 * 2048 or 4096)."""
    grid = 256 * waves_per_cu // 4
    if out is None:
        out = torch.empty(grid * 256, dtype=torch.float32, device=device)
    _check(LIB.inv_mfma_rate_probe(int(shape), int(iters), int(waves_per_cu), _p(out),
                                   torch.cuda.current_stream(out.device).cuda_stream), "inv_mfma_rate_probe")
    return out
