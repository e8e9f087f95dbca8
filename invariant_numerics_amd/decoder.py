"""Llama-shaped decoder assembled from the library's C-ABI calls (LayerCast setting:
BF16 weights, FP32 activations and KV cache, every reduction in the fixed order).

Two ways to score a batch of sequences that must give the same bits at every position:
  * ``prefill``: token blocks of all sequences at once (rows ordered (sequence, position)),
    every layer through fixed_order_gemm / rmsnorm / rope_kv_append / attention_prefill;
  * ``decode_step``: one token per sequence (M = batch), attention_decode over the cache.
Every op is row-independent and chunk boundaries are absolute key positions, so token
blocking, batch size and prefill-vs-decode do not change a row's bits.

Activation storage policy ``act``: "fp32" (LayerCast: every activation and the KV cache in
FP32, fused residual and gated epilogues) or "bf16" / "fp16": every activation tensor an
unfused implementation stores between operations (embedding, norm outputs, projection outputs,
rotated q and k and the cache, attention output, the SwiGLU product, residual sums) is rounded
to that format; each operation still computes in FP32 from the rounded values.  These are the
low-precision bodies of the cross-precision comparison ("Greedy Decoding Is Not
Precision-Invariant", abstract).  Weights and the LM head are the same under every policy.

Weight layouts (nn.Linear): wqkv [(Hq+2Hkv)D, H] = q rows | k rows | v rows; wo [H, Hq D];
w13 [2F, H] = gate rows | up rows (held on the device with gate and up rows interleaved for
the gated projection); w2 [H, F]; whead [V, H]; emb [V, H]; RoPE tables
cos/sin [Tmax, D/2] fp32.
"""
import numpy as np
import torch

from . import binding as inv


def _interleave_gate_up(w13):
    """[gate rows | up rows] -> rows (gate 0, up 0, gate 1, up 1, ...), the layout the gated
    projection reads (a row permutation: every output is computed exactly as before)."""
    F = w13.shape[0] // 2
    out = np.empty_like(w13)
    out[0::2] = w13[:F]
    out[1::2] = w13[F:]
    return out


def _to_dev_bf16(a, dev):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)


class Decoder:
    def __init__(self, model, device="cuda", batch=1, tmax=None, tau=0.1, eps=1e-5, act="fp32"):
        if act not in inv.ACT_FORMATS:
            raise inv.InvError("unknown activation format %r" % (act,))
        self.act = act
        cfg = model["cfg"]
        self.cfg = cfg
        self.H, self.Hq, self.Hkv, self.D = cfg["hidden"], cfg["hq"], cfg["hkv"], cfg["d"]
        self.F, self.V, self.L = cfg["ffn"], cfg["vocab"], cfg["layers"]
        self.dev = torch.device(device)
        self.tau = float(np.float32(tau))
        self.eps = float(np.float32(eps))
        self.emb = _to_dev_bf16(model["emb"], self.dev)
        self.whead = _to_dev_bf16(model["whead"], self.dev)
        self.gf = _to_dev_bf16(model["gf"], self.dev)
        # the fused gated projection (FP32 policy) reads gate and up rows interleaved; the
        # rounded policies store gate and up outputs, so they keep the [gate | up] layout
        inter = act == "fp32"
        self.layers = [{k: _to_dev_bf16(_interleave_gate_up(v) if (k == "w13" and inter) else v, self.dev)
                        for k, v in layer.items()} for layer in model["layers"]]
        self.cos = torch.from_numpy(np.ascontiguousarray(model["cos"])).to(self.dev)
        self.sin = torch.from_numpy(np.ascontiguousarray(model["sin"])).to(self.dev)
        self.tmax = int(tmax if tmax is not None else self.cos.shape[0])
        assert self.cos.shape[0] >= self.tmax
        self.batch = int(batch)
        self.kc = [torch.zeros((batch, self.Hkv, self.tmax, self.D), dtype=torch.float32, device=self.dev)
                   for _ in range(self.L)]
        self.vc = [torch.zeros_like(k) for k in self.kc]
        # optional measurement hook: when a list, each body projection appends
        # (start event, end event, algorithmic flops, algorithmic bytes) recorded on its
        # launch stream
        self.gemm_events = None

    def _gemm(self, X, W, R=None, out=None, gated=False):
        def call():
            if gated:
                return inv.inv_gated_gemm(X, W, out=out)
            return inv.inv_fixed_order_gemm(X, W, R=R, out=out)
        ev = self.gemm_events
        if ev is None:
            return call()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        y = call()
        e.record()
        M, K = X.shape
        N = W.shape[0]
        # algorithmic bytes: X and W read once, Y written once (R read once when given)
        nbytes = 4 * M * K + 2 * N * K + 4 * M * (N // 2 if gated else N) * (2 if R is not None else 1)
        ev.append((s, e, 2.0 * M * N * K, float(nbytes)))
        return y

    # one pass of the decoder body over rows (seq[m], pos[m]); attention via `attend`
    def _body(self, ids, seq, pos, attend):
        if self.act != "fp32":
            return self._body_rounded(ids, seq, pos, attend)
        H, Hq, Hkv, D, F = self.H, self.Hq, self.Hkv, self.D, self.F
        M = ids.numel()
        x = inv.inv_embed(ids, self.emb)
        n = torch.empty_like(x)
        q = torch.empty((M, Hq, D), dtype=torch.float32, device=self.dev)
        # up to four rows (decode): RoPE with the KV append runs in the QKV projection's epilogue;
        # for one row each RMSNorm also runs in the prologue of the projection that reads it
        # (same bits, one and three launches fewer per layer; with more rows the prologue,
        # which walks the rows in turn, costs more than the norm's launch)
        fused = M <= 4 and D == 128 and self.gemm_events is None
        fnorm = fused and M == 1
        for li, w in enumerate(self.layers):
            if fnorm:
                inv.inv_rmsnorm_qkv_rope_kv_append(x, w["g1"], w["wqkv"], Hq, Hkv, D, seq, pos, self.cos,
                                                   self.sin, q, self.kc[li], self.vc[li], eps=self.eps)
            elif fused:
                inv.inv_rmsnorm(x, w["g1"], self.eps, out=n)
                inv.inv_qkv_rope_kv_append(n, w["wqkv"], Hq, Hkv, D, seq, pos, self.cos, self.sin, q,
                                           self.kc[li], self.vc[li])
            else:
                inv.inv_rmsnorm(x, w["g1"], self.eps, out=n)
                qkv = self._gemm(n, w["wqkv"])
                inv.inv_rope_kv_append(qkv, Hq, Hkv, D, seq, pos, self.cos, self.sin, q, self.kc[li], self.vc[li])
                del qkv
            att = attend(q, li)
            self._gemm(att.view(M, Hq * D), w["wo"], R=x, out=x)
            del att
            if fnorm:
                h = inv.inv_rmsnorm_gemm(x, w["g2"], w["w13"], eps=self.eps, gated=True)
            else:
                inv.inv_rmsnorm(x, w["g2"], self.eps, out=n)
                h = self._gemm(n, w["w13"], gated=True)     # silu(gate) * up, [M, F]
            self._gemm(h, w["w2"], R=x, out=x)
            del h
        inv.inv_rmsnorm(x, self.gf, self.eps, out=n)
        return n

    # the same body with every stored activation rounded to self.act (unfused epilogues:
    # projection outputs are stored, then added to the residual)
    def _body_rounded(self, ids, seq, pos, attend):
        H, Hq, Hkv, D, F = self.H, self.Hq, self.Hkv, self.D, self.F
        fmt = self.act

        def R(t):
            return inv.inv_round_activations(t, fmt, out=t)

        M = ids.numel()
        x = R(inv.inv_embed(ids, self.emb))
        n = torch.empty_like(x)
        q = torch.empty((M, Hq, D), dtype=torch.float32, device=self.dev)
        for li, w in enumerate(self.layers):
            R(inv.inv_rmsnorm(x, w["g1"], self.eps, out=n))
            qkv = R(self._gemm(n, w["wqkv"]))
            inv.inv_rope_kv_append(qkv, Hq, Hkv, D, seq, pos, self.cos, self.sin, q, self.kc[li], self.vc[li],
                                   fmt=fmt)
            del qkv
            att = R(attend(q, li).view(M, Hq * D))
            o = R(self._gemm(att, w["wo"]))
            del att
            R(inv.inv_add(x, o, out=x))
            del o
            R(inv.inv_rmsnorm(x, w["g2"], self.eps, out=n))
            gu = R(self._gemm(n, w["w13"]))             # [gate | up], [M, 2F]
            h = R(inv.inv_swiglu(gu[:, :F], gu[:, F:]))
            del gu
            y = R(self._gemm(h, w["w2"]))
            del h
            R(inv.inv_add(x, y, out=x))
            del y
        R(inv.inv_rmsnorm(x, self.gf, self.eps, out=n))
        return n

    def prefill(self, tokens, block=2048, lm_rows=None):
        """Score tokens [B, T] (device int32, B <= batch): returns dict of [B, T-1] device
        tensors (logprob, margin, top1, top2, recomputed) for positions 0..T-2."""
        B, T = tokens.shape
        assert B <= self.batch and T <= self.tmax
        out = {k: torch.empty((B, T - 1), dtype=dt, device=self.dev) for k, dt in
               (("logprob", torch.float32), ("margin", torch.float32), ("top1", torch.int32),
                ("top2", torch.int32), ("recomputed", torch.uint8))}
        tgt_all = torch.zeros((B, T), dtype=torch.int32, device=self.dev)
        tgt_all[:, :T - 1] = tokens[:, 1:]
        for q0 in range(0, T, block):
            q1 = min(T, q0 + block)
            nb = q1 - q0
            ids = tokens[:, q0:q1].contiguous().view(-1)
            seq = torch.arange(B, dtype=torch.int32, device=self.dev).repeat_interleave(nb)
            pos = torch.arange(q0, q1, dtype=torch.int32, device=self.dev).repeat(B)

            def attend(q, li, q0=q0, nb=nb):
                return inv.inv_attention_prefill(q.view(B, nb, self.Hq, self.D), self.kc[li][:B],
                                                 self.vc[li][:B], q_start=q0)

            hn = self._body(ids, seq, pos, attend)
            tg = tgt_all[:, q0:q1].contiguous().view(-1)
            r = self._lmhead(hn, tg, lm_rows)
            nscore = min(q1, T - 1) - q0
            if nscore > 0:
                for k in out:
                    out[k][:, q0:q0 + nscore] = r[k].view(B, nb)[:, :nscore]
        return out

    def _lmhead(self, hn, tg, lm_rows=None):
        M = hn.shape[0]
        step = M if not lm_rows else int(lm_rows)
        if step >= M:
            return inv.inv_lmhead_logprob_top2(hn, self.whead, tg, self.tau)
        parts = [inv.inv_lmhead_logprob_top2(hn[s:s + step], self.whead, tg[s:s + step], self.tau)
                 for s in range(0, M, step)]
        return {k: torch.cat([p[k] for p in parts]) for k in parts[0]}

    def decode_step(self, tok, pos, target):
        """One token per sequence: tok, pos, target int32 [B] (device).  Writes the cache at
        pos and returns the LM-head outputs for those positions (dict of [B] tensors)."""
        B = tok.numel()
        seq = torch.arange(B, dtype=torch.int32, device=self.dev)

        def attend(q, li):
            return inv.inv_attention_decode(q, self.kc[li][:B], self.vc[li][:B], pos)

        hn = self._body(tok, seq, pos, attend)
        return inv.inv_lmhead_logprob_top2(hn, self.whead, target, self.tau)

    def decode_graph(self, B=None):
        """Capture one decode step (batch B) in a HIP graph.  Returns step(tok, pos, target)
        that copies the int32 [B] inputs into the graph's static buffers, replays it and returns
        the graph's output tensors (valid until the next replay).  Every kernel of the step reads
        token, position and target from device memory, and none of them issues a memset, so one
        capture serves every position."""
        B = self.batch if B is None else int(B)
        st_tok = torch.zeros(B, dtype=torch.int32, device=self.dev)
        # position -1 during warm-up: rope_kv_append skips rows outside the cache and decode
        # attention reads nothing for them, so the warm-up leaves the KV cache untouched
        st_pos = torch.full((B,), -1, dtype=torch.int32, device=self.dev)
        st_tgt = torch.zeros(B, dtype=torch.int32, device=self.dev)
        side = torch.cuda.Stream(device=self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            self.decode_step(st_tok, st_pos, st_tgt)          # warm-up outside the capture
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize(self.dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            st_out = self.decode_step(st_tok, st_pos, st_tgt)

        def step(tok, pos, target):
            st_tok.copy_(tok)
            st_pos.copy_(pos)
            st_tgt.copy_(target)
            graph.replay()
            return st_out

        step.graph = graph
        return step

    def decode_graph_steps(self, K, B=None):
        """Capture K consecutive decode steps (batch B) in one HIP graph.  Returns
        run(tok, pos, target) taking int32 [K, B] inputs (step k reads row k: the token, position
        and target of every sequence at that step), which copies them into the graph's static
        buffers, replays the K steps and returns their K output dicts (valid until the next
        replay).  The steps are the single-step graph's kernels in sequence; one replay pays the
        input copies and the graph launch once for K steps."""
        B = self.batch if B is None else int(B)
        K = int(K)
        st_tok = torch.zeros((K, B), dtype=torch.int32, device=self.dev)
        st_pos = torch.full((K, B), -1, dtype=torch.int32, device=self.dev)   # warm-up: no cache writes
        st_tgt = torch.zeros((K, B), dtype=torch.int32, device=self.dev)
        side = torch.cuda.Stream(device=self.dev)
        side.wait_stream(torch.cuda.current_stream(self.dev))
        with torch.cuda.stream(side):
            self.decode_step(st_tok[0], st_pos[0], st_tgt[0])
        torch.cuda.current_stream(self.dev).wait_stream(side)
        torch.cuda.synchronize(self.dev)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            st_out = [self.decode_step(st_tok[k], st_pos[k], st_tgt[k]) for k in range(K)]

        def run(tok, pos, target):
            st_tok.copy_(tok)
            st_pos.copy_(pos)
            st_tgt.copy_(target)
            graph.replay()
            return st_out

        run.graph = graph
        return run
