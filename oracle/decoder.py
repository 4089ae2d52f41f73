"""A small dense decoder for the weight-bearing ODA step, in float64 (oracle side).

ODA summary page, "Approach": at every token the Local pass runs first; the
recall head reads [h_{t-1}, E(x_t), h^L_t] -- the previously selected hidden
state, the current token's embedding and the final hidden state of this Local
pass -- and when q_t > theta the step is recomputed from the same prior state
with Full attention and that pass is selected; the current position's KV of
the selected pass is committed to the preserved history. With real layers the
recall pass's keys and values differ from the Local pass's from the second
layer on (their inputs went through different attention), which is what this
model makes visible.

The pages name the backbones (Qwen3 family) but not their layer structure.
The layer here is the Qwen3-family decoder layer as published, with random
weights (reading, stated in the design notes):

    x  = RMSNorm(h) * g_attn
    q, k, v = split(W_qkv x)                 per head: q, k RMS-normalised
    q, k = RoPE(q, pos), RoPE(k, pos)         rotate-half pairs (i, i + D/2),
                                              angle pos * base^(-2i/D)
    o  = attention of q over the view, with (k, v) committed at pos = n - 1
    h  = h + W_o o
    x  = RMSNorm(h) * g_mlp
    h  = h + W_down (SiLU(W_gate x) * (W_up x))

and the final hidden state is RMSNorm(h) * g_final. Weights are bf16 (the
values used are their exact bf16 values); activations are float64; the
committed key and value are the bf16 roundings of the float64 results. Inputs
come from a token stream (no LM head is evaluated).
"""

import math

import numpy as np

from . import oda, recall
from .bf16 import bf16_bits_to_f64, f64_to_bf16_bits


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(g, dtype=np.float64)


def rope(x, pos, base):
    """Rotary position embedding of rows x [H][D] at position pos (rotate-half)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * base ** (-2.0 * i / D)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


class DecoderShape:
    def __init__(self, layers, hidden, q_heads, kv_heads, intermediate, vocab, recall_hidden, head_dim=128,
                 eps=1e-6, rope_base=1.0e6):
        self.layers, self.hidden, self.q_heads, self.kv_heads = layers, hidden, q_heads, kv_heads
        self.intermediate, self.vocab, self.recall_hidden = intermediate, vocab, recall_hidden
        self.head_dim, self.eps, self.rope_base = head_dim, eps, rope_base


class Decoder:
    """Weights given as bf16 bit arrays (uint16), widened exactly to float64.

    w: dict with 'emb' [V][d], 'g_final' [d], 'W1' [hr][3d] (fp32 recall head:
    'W1', 'b1', 'w2', 'b2' as float arrays), and per layer l: 'qkv.l'
    [(Hq+2Hkv)D][d], 'g_attn.l' [d], 'g_q.l' [D], 'g_k.l' [D], 'o.l' [d][Hq D],
    'g_mlp.l' [d], 'gu.l' [2I][d] (gate rows then up rows), 'down.l' [d][I].
    """

    def __init__(self, shape, w):
        self.s = shape
        self.w = {}
        for k, v in w.items():
            v = np.asarray(v)
            self.w[k] = bf16_bits_to_f64(v) if v.dtype == np.uint16 else v.astype(np.float64)

    def layer(self, l, h, hist_k, hist_v, n, full, scale, sinks, window):
        s, w = self.s, self.w
        D, Hq, Hkv = s.head_dim, s.q_heads, s.kv_heads
        x = rms_norm(h, w["g_attn.%d" % l], s.eps)
        qkv = w["qkv.%d" % l] @ x
        q = qkv[:Hq * D].reshape(Hq, D)
        k = qkv[Hq * D:(Hq + Hkv) * D].reshape(Hkv, D)
        v = qkv[(Hq + Hkv) * D:].reshape(Hkv, D)
        q = rope(rms_norm(q, w["g_q.%d" % l], s.eps), n - 1, s.rope_base)
        k = rope(rms_norm(k, w["g_k.%d" % l], s.eps), n - 1, s.rope_base)
        kb, vb = f64_to_bf16_bits(k), f64_to_bf16_bits(v)
        if full:
            o = oda.full_pass(q, kb, vb, hist_k, hist_v, n, scale)
        else:
            o = oda.local_pass(q, kb, vb, hist_k, hist_v, n, scale, sinks, window)
        h = h + w["o.%d" % l] @ o.reshape(-1)
        x = rms_norm(h, w["g_mlp.%d" % l], s.eps)
        gu = w["gu.%d" % l] @ x
        I = s.intermediate
        return h + w["down.%d" % l] @ (silu(gu[:I]) * gu[I:])

    def forward(self, token, hist, n, full, scale=None, sinks=4, window=2048):
        """One pass over all layers for the token at position n-1; hist[l] = (k_bits,
        v_bits) is updated in place (commit). Returns the final hidden state."""
        scale = 1.0 / math.sqrt(self.s.head_dim) if scale is None else scale
        h = self.w["emb"][int(token)].copy()
        for l in range(self.s.layers):
            h = self.layer(l, h, hist[l][0], hist[l][1], n, full, scale, sinks, window)
        return rms_norm(h, self.w["g_final"], self.s.eps)

    def oda_step(self, token, h_prev, hist, n, theta=0.0, decide=None, **kw):
        """One ODA step: Local pass, recall head, Full pass when q_t > theta.

        Returns (h_selected, gate, q_t, h_local). `decide`, when given, maps q_t to
        the decision (a test adopts the device's decision inside its tolerance band).
        """
        hL = self.forward(token, hist, n, False, **kw)
        x = recall.concat_inputs(h_prev, self.w["emb"][int(token)], hL)
        q_t = recall.recall_score(x, self.w["W1"], self.w["b1"], self.w["w2"], self.w["b2"])
        g = recall.gate(q_t, theta) if decide is None else decide(q_t)
        if g:
            return self.forward(token, hist, n, True, **kw), True, q_t, hL
        return hL, False, q_t, hL
