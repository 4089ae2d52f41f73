"""Weight-bearing ODA decode step: the library calls that run one token through a
small dense decoder with On-Demand Attention, in order.

On-Demand Attention summary page, "Approach": at every token the Local pass runs
first through all layers; the recall head reads [h_{t-1}, E(x_t), h^L_t] (the
previously selected final hidden state, the token embedding and this Local pass's
final hidden state); when q_t > theta the whole model reruns from the same prior
state with Full attention and that pass is selected, its keys and values being the
ones committed. Here every launch of the recall pass carries the gate as its
selector, so the step is one fixed sequence of launches (a HIP graph) with no host
round trip ("Developer perspective").

Layer (Qwen3-family): sk_gemv W_qkv (RMSNorm prologue; the raw q/k/v projection) ->
oda_decode_local_qkv / oda_decode_full_qkv (per-head q/k norm and RoPE applied while the
attention stages its operands; the bf16 k/v candidate committed at n-1) -> sk_gemv W_o
(+ residual) -> sk_gemv W_gate|up (RMSNorm prologue, SwiGLU epilogue) -> sk_gemv W_down
(+ residual). With fuse_qk=False the per-head finish runs as its own launch
(sk_qkv_rope) before oda_decode_local / oda_decode_full.

This module only sequences library calls; it computes nothing itself.
"""

import math

import torch

from . import ops


class DecoderShape:
    def __init__(self, layers, hidden, q_heads, kv_heads, intermediate, vocab, recall_hidden, eps=1e-6,
                 rope_base=1.0e6):
        self.layers, self.hidden, self.q_heads, self.kv_heads = layers, hidden, q_heads, kv_heads
        self.intermediate, self.vocab, self.recall_hidden = intermediate, vocab, recall_hidden
        self.eps, self.rope_base = eps, rope_base


class ODADecoder:
    """Device weights, paged caches and the step buffers of a batch-1 decoder.

    weights: dict of GPU tensors -- 'emb' bf16 [V][d], 'g_final' bf16 [d], recall head
    'W1' fp32 [hr][3d], 'b1' [hr], 'w2' [hr], 'b2' [1]; per layer l: 'qkv.l' bf16
    [(Hq+2Hkv)128][d], 'g_attn.l' [d], 'g_q.l' [128], 'g_k.l' [128], 'o.l' [d][Hq 128],
    'g_mlp.l' [d], 'gu.l' [2I][d], 'down.l' [d][I].
    caches: one ops.PagedKVCache per layer (batch 1), sharing seq_lens.
    """

    def __init__(self, shape, weights, caches, sinks=4, window=2048, scale=None, device="cuda",
                 local_only=(), fuse_qk=True):
        s = shape
        self.fuse_qk = fuse_qk
        self.s, self.w, self.caches = s, weights, caches
        self.sinks, self.window = sinks, window
        self.scale = 1.0 / math.sqrt(ops.HEAD_DIM) if scale is None else scale
        self.seq_lens = caches[0].seq_lens
        self.local_only = frozenset(local_only)
        f32, dev = torch.float32, device
        d, D = s.hidden, ops.HEAD_DIM
        self.token = torch.zeros(1, dtype=torch.int32, device=dev)
        self.h_local = torch.zeros(d, dtype=f32, device=dev)
        self.h_full = torch.zeros(d, dtype=f32, device=dev)
        self.final_full = torch.zeros(d, dtype=f32, device=dev)
        self.x_rec = torch.zeros(3 * d, dtype=f32, device=dev)  # [h_{t-1} | E(x_t) | h^L_t]
        self.q = torch.zeros((1, s.q_heads, D), dtype=f32, device=dev)
        self.k = torch.zeros((1, s.kv_heads, D), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros_like(self.k)
        self.attn = torch.zeros((1, s.q_heads, D), dtype=f32, device=dev)
        self.act = torch.zeros(s.intermediate, dtype=f32, device=dev)  # SiLU(gate) * up
        self.qkv_raw = torch.zeros((s.q_heads + 2 * s.kv_heads) * D, dtype=f32, device=dev)
        self.qscore = torch.zeros(1, dtype=f32, device=dev)
        self.gate = torch.zeros(1, dtype=torch.int32, device=dev)
        self.ws = ops.workspace(1, s.q_heads, dev)

    @property
    def h_prev(self):
        """The selected final hidden state of the last step (the recall head's h_{t-1})."""
        return self.x_rec[:self.s.hidden]

    @property
    def h_local_final(self):
        return self.x_rec[2 * self.s.hidden:]

    def _layer(self, l, h, full, sel):
        s, w = self.s, self.w
        use_full = full and l not in self.local_only
        if self.fuse_qk:
            ops.gemv(w["qkv.%d" % l], h, self.qkv_raw, prologue=ops.PRO_RMSNORM, gamma=w["g_attn.%d" % l], eps=s.eps,
                     sel=sel)
            qk = dict(eps=s.eps, rope_base=s.rope_base, scale=self.scale, sel=sel, sel_value=1, out=self.attn,
                      ws=self.ws)
            if use_full:
                ops.oda_decode_full_qkv(self.qkv_raw, w["g_q.%d" % l], w["g_k.%d" % l], self.caches[l], **qk)
            else:
                ops.oda_decode_local_qkv(self.qkv_raw, w["g_q.%d" % l], w["g_k.%d" % l], self.caches[l],
                                         sinks=self.sinks, window=self.window, **qk)
        else:
            ops.qkv_rope(w["qkv.%d" % l], h, w["g_attn.%d" % l], w["g_q.%d" % l], w["g_k.%d" % l], s.q_heads,
                         s.kv_heads, self.seq_lens, self.qkv_raw, self.q, self.k, self.v, eps=s.eps,
                         rope_base=s.rope_base, sel=sel, sel_value=1)
            if use_full:
                ops.oda_decode_full(self.q, self.caches[l], self.k, self.v, self.scale, sel=sel, sel_value=1,
                                    out=self.attn, ws=self.ws)
            else:
                ops.oda_decode_local(self.q, self.caches[l], self.k, self.v, self.sinks, self.window, self.scale,
                                     sel=sel, sel_value=1, out=self.attn, ws=self.ws)
        ops.gemv(w["o.%d" % l], self.attn.view(-1), h, residual=h, sel=sel)
        ops.gemv(w["gu.%d" % l], h, self.act, prologue=ops.PRO_RMSNORM, gamma=w["g_mlp.%d" % l], eps=s.eps,
                 epilogue=ops.EPI_SWIGLU, sel=sel)
        ops.gemv(w["down.%d" % l], self.act, h, residual=h, sel=sel)

    def local_pass(self):
        d = self.s.hidden
        ops.embed(self.w["emb"], self.token, self.h_local, out2=self.x_rec[d:2 * d])
        for l in range(self.s.layers):
            self._layer(l, self.h_local, False, None)
        ops.rmsnorm(self.h_local, self.w["g_final"], self.h_local_final, eps=self.s.eps)

    def recall_gate(self, theta=0.0):
        w = self.w
        ops.oda_recall_score(self.x_rec.view(1, -1), w["W1"], w["b1"], w["w2"], w["b2"], theta, q_out=self.qscore,
                             gate_out=self.gate, ws=self.ws)

    def recall_pass(self, gated=True):
        sel = self.gate if gated else None
        ops.embed(self.w["emb"], self.token, self.h_full, sel=sel)
        for l in range(self.s.layers):
            self._layer(l, self.h_full, True, sel)
        ops.rmsnorm(self.h_full, self.w["g_final"], self.final_full, eps=self.s.eps, sel=sel)

    def step(self, theta=0.0):
        """One ODA step for the token in self.token at n = seq_lens[0]."""
        self.local_pass()
        self.recall_gate(theta)
        self.recall_pass(gated=True)
        ops.select(self.gate, self.final_full, self.h_local_final, self.h_prev)

    def always_full_step(self):
        """Baseline: every step runs the model once with Full attention."""
        self.recall_pass(gated=False)
