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
