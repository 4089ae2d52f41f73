"""Cost counters for the decode views (oracle side).

ODA summary page, "Approach", cost model: the Local pass costs a fixed
l = s + w keys per step, the Full pass grows linearly with the history length
n, and the average saving follows from the Full-call rate rho.

Per attention layer-step over a key set S with Hq query heads, Hkv KV heads and
head dimension D:

    attention FLOPs = 4 * Hq * D * |S|      (QK^T and PV, 2 FLOPs per MAC)
    KV bytes        = |S| * Hkv * D * 2 (K and V) * 2 (bf16)
"""

from fractions import Fraction

from . import keysets


def local_size(n, sinks=4, window=2048):
    return int(keysets.local_keys(n, sinks, window).size)


def attention_flops(num_keys, Hq, D):
    return 4 * Hq * D * num_keys


def kv_bytes(num_keys, Hkv, D):
    return num_keys * Hkv * D * 2 * 2


def local_over_full(n, sinks=4, window=2048):
    """|S_L| / |S_F| as an exact fraction."""
    return Fraction(local_size(n, sinks, window), n)


def oda_over_full(ns, recall_flags, sinks=4, window=2048):
    """Attention-only cost of ODA over always-Full for a sequence of steps with
    key counts ``ns``: Local every step, plus Full on recall steps."""
    oda = sum(local_size(n, sinks, window) + (n if r else 0) for n, r in zip(ns, recall_flags))
    full = sum(ns)
    return Fraction(oda, full)


# ---------------------------------------------------------------- whole-model accounting
#
# ODA summary page, "Main results", efficiency bullet: at 128K input, 1K output and
# about 12.5 % Full calls, ODA spends 24.26 % of the main decoding FLOPs of always-Full
# decoding, and vLLM's throughput goes from 75.54 to 149.52 tokens/s (1.98x). The same
# page's "Limitations" bullet places the speed and FLOP measurements on Qwen3-1.7B.
#
# A decode step of a dense decoder costs, per token:
#   dense FLOPs   = 2 * (per-layer projection and MLP weights + LM-head weights)
#   attention     = layers * 4 * Hq * D * |S|          (per key, as above)
#   recall head   = 2 * its parameter count             (a GEMV stack; the page gives
#                                                        28,325,889 parameters)
# An ODA step runs the Local pass (dense + attention over the Local view) and the
# recall head every step, and on a recall step the whole model again with Full
# attention ("Approach": the step is recomputed from the same prior state).
# Always-Full decoding runs dense + attention over all n keys once per step.
#
# Byte counts use the same structure: weights (bf16) are read once per pass, the
# recall head's fp32 weights once per step, and the KV bytes of the attended keys.

class DenseShape:
    """Sizes of a dense decoder: attention heads, a gated (three-matrix) MLP and an
    LM head of vocab x hidden. Norm, rotary and embedding-lookup costs are omitted."""

    def __init__(self, layers, hidden, q_heads, kv_heads, head_dim, intermediate, vocab, recall_params=0):
        self.layers, self.hidden = layers, hidden
        self.q_heads, self.kv_heads, self.head_dim = q_heads, kv_heads, head_dim
        self.intermediate, self.vocab, self.recall_params = intermediate, vocab, recall_params

    def layer_params(self):
        h, d = self.hidden, self.head_dim
        attn = h * self.q_heads * d + 2 * h * self.kv_heads * d + self.q_heads * d * h
        return attn + 3 * h * self.intermediate

    def params(self):
        """Weights read per pass (the LM head shares the embedding matrix)."""
        return self.layers * self.layer_params() + self.vocab * self.hidden


def dense_flops(m):
    return 2 * m.params()


def model_attention_flops(m, num_keys):
    return m.layers * attention_flops(num_keys, m.q_heads, m.head_dim)


def step_flops_full(m, n):
    return dense_flops(m) + model_attention_flops(m, n)


def step_flops_oda(m, n, recalled, sinks=4, window=2048):
    cost = dense_flops(m) + model_attention_flops(m, local_size(n, sinks, window)) + 2 * m.recall_params
    if recalled:
        cost += step_flops_full(m, n)
    return cost


def decode_flops_ratio(m, ns, recall_flags, sinks=4, window=2048):
    """Whole-model decode FLOPs of ODA over always-Full, exact fraction."""
    oda = sum(step_flops_oda(m, n, r, sinks, window) for n, r in zip(ns, recall_flags))
    full = sum(step_flops_full(m, n) for n in ns)
    return Fraction(oda, full)


def step_bytes_full(m, n, weight_bytes=2):
    return m.params() * weight_bytes + m.layers * kv_bytes(n, m.kv_heads, m.head_dim)


def step_bytes_oda(m, n, recalled, sinks=4, window=2048, weight_bytes=2):
    cost = (m.params() * weight_bytes + m.layers * kv_bytes(local_size(n, sinks, window), m.kv_heads, m.head_dim)
            + 4 * m.recall_params)
    if recalled:
        cost += step_bytes_full(m, n, weight_bytes)
    return cost


def decode_bytes_ratio(m, ns, recall_flags, sinks=4, window=2048):
    """Whole-model bytes moved per decoded token, always-Full over ODA (an upper bound
    on the speedup of a bandwidth-bound decoder)."""
    full = sum(step_bytes_full(m, n) for n in ns)
    oda = sum(step_bytes_oda(m, n, r, sinks, window) for n, r in zip(ns, recall_flags))
    return Fraction(full, oda)
