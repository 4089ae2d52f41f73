"""Seeded weights, token stream and history of the weight-bearing decode workloads.

A decoder workload is a small dense decoder of the Qwen3 family (random weights:
projections N(0, sigma^2) in bf16, norm gains 1 + N(0, 0.1^2) in bf16, token
embeddings N(0, 1) in bf16, an fp32 recall head 3d -> hr -> 1 with N(0, 0.02^2)
weights and zero biases), a seeded token stream and a synthetic KV history per
layer. Every tensor is one synth.rng stream keyed by (workload id, C_WEIGHT, index
of the tensor), so the host (for the oracle) and the device fill produce the same
bits. Only inputs are generated here; nothing of the method is computed.
"""

import numpy as np
import torch

from . import rng
from .workloads import BLOCK, C_KHIST, C_TOKENS, C_VHIST, np_rng

C_WEIGHT = 30
D = 128


class DecoderWorkload:
    def __init__(self, wid, name, layers, hidden, q_heads, kv_heads, intermediate, vocab, recall_hidden, H0,
                 steps, sigma=0.02, sinks=4, window=2048, theta=0.0, eps=1e-6, rope_base=1.0e6):
        self.wid, self.name = wid, name
        self.layers, self.hidden, self.q_heads, self.kv_heads = layers, hidden, q_heads, kv_heads
        self.intermediate, self.vocab, self.recall_hidden = intermediate, vocab, recall_hidden
        self.H0, self.steps, self.sigma = H0, steps, sigma
        self.sinks, self.window, self.theta, self.eps, self.rope_base = sinks, window, theta, eps, rope_base
        self.max_blocks = -(-(H0 + steps) // BLOCK)
        self.tokens = np_rng(wid, C_TOKENS).integers(0, vocab, size=steps).astype(np.int32)

    # (name, shape, kind) in a fixed order; the index is the stream unit
    def tensors(self):
        d, I, Hq, Hkv, hr = self.hidden, self.intermediate, self.q_heads, self.kv_heads, self.recall_hidden
        out = [("emb", (self.vocab, d), "emb"), ("g_final", (d,), "gain"),
               ("W1", (hr, 3 * d), "head"), ("w2", (hr,), "head"), ("b1", (hr,), "zero"), ("b2", (1,), "zero")]
        for l in range(self.layers):
            out += [("qkv.%d" % l, ((Hq + 2 * Hkv) * D, d), "mat"), ("g_attn.%d" % l, (d,), "gain"),
                    ("g_q.%d" % l, (D,), "gain"), ("g_k.%d" % l, (D,), "gain"), ("o.%d" % l, (d, Hq * D), "mat"),
                    ("g_mlp.%d" % l, (d,), "gain"), ("gu.%d" % l, (2 * I, d), "mat"),
                    ("down.%d" % l, (d, I), "mat")]
        return out

    def key(self, unit):
        return rng.mix_key(self.wid, C_WEIGHT, unit)

    def _host(self, unit, shape, kind):
        n = int(np.prod(shape))
        if kind == "mat":
            return rng.normal_bf16(self.key(unit), 0, n, rng.unit_scale(self.sigma)).reshape(shape)
        if kind == "emb":
            return rng.normal_bf16(self.key(unit), 0, n, rng.unit_scale(1.0)).reshape(shape)
        if kind == "gain":
            g = np.float32(1.0) + rng.normal_f32(self.key(unit), 0, n, rng.unit_scale(0.1))
            return rng.f32_to_bf16_bits(g.astype(np.float32)).reshape(shape)
        if kind == "head":
            return rng.normal_f32(self.key(unit), 0, n, rng.unit_scale(0.02)).reshape(shape)
        return np.zeros(shape, np.float32)

    def host_weights(self):
        """Every tensor on the host: uint16 bf16 bits, or float32 for the recall head."""
        return {name: self._host(u, shape, kind) for u, (name, shape, kind) in enumerate(self.tensors())}

    def device_weights(self, device="cuda"):
        """The same tensors on the device; large matrices are filled there."""
        from .device import fill_normal_
        out = {}
        for u, (name, shape, kind) in enumerate(self.tensors()):
            if kind in ("mat", "emb"):
                t = torch.empty(shape, dtype=torch.bfloat16, device=device)
                fill_normal_(t, self.key(u), 0, self.sigma if kind == "mat" else 1.0)
            else:
                a = self._host(u, shape, kind)
                if a.dtype == np.uint16:
                    t = torch.as_tensor(a.view(np.int16), device=device).view(torch.bfloat16)
                else:
                    t = torch.as_tensor(a, device=device)
            out[name] = t
        return out

    def hist_key(self, kind, layer):
        return rng.mix_key(self.wid, C_KHIST if kind == "k" else C_VHIST, layer)

    def hist_bits(self, kind, layer, start, count):
        e = self.kv_heads * D
        return rng.normal_bf16(self.hist_key(kind, layer), start * e, count * e, rng.unit_scale()).reshape(
            count, self.kv_heads, D)


def decoder_small(steps=12, H0=3000):
    """Parity-sized: 3 layers, hidden 512, 4 q / 2 kv heads, MLP 1024, vocab 512, history
    3000 (beyond the Local view), recall head 1536 -> 64 -> 1."""
    return DecoderWorkload(7, "decoder_small", layers=3, hidden=512, q_heads=4, kv_heads=2, intermediate=1024,
                           vocab=512, recall_hidden=64, H0=H0, steps=steps)


def decoder_qwen3_1_7b(H0, steps):
    """Qwen3-1.7B's dense shape (28 layers, hidden 2048, 16 q / 8 kv heads of 128, MLP
    6144, vocabulary 151936) with random weights, recall head 6144 -> 512 -> 1."""
    return DecoderWorkload(8, "decoder_qwen3_1.7b", layers=28, hidden=2048, q_heads=16, kv_heads=8,
                           intermediate=6144, vocab=151936, recall_hidden=512, H0=H0, steps=steps)
