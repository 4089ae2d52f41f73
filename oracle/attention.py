"""Single-token decode attention over a key set, in float64 (oracle side).

For query head h with KV head g = floor(h * Hkv / Hq) (contiguous grouping of
query heads onto KV heads, the usual grouped-query convention; the pages do not
fix it), and a key set S:

    z_j = scale * <q_h, k_{g,j}>          for j in S
    m   = max_j z_j
    p_j = exp(z_j - m) / sum_{i in S} exp(z_i - m)
    o_h = sum_{j in S} p_j * v_{g,j}

This is plain scaled-dot-product softmax attention. ODA and DA change which
keys are read, not how attention is computed (ODA summary page, "Approach":
Local and Full are two views of the same attention; DA review page, section 3:
the existing attention kernel is reused unmodified on the kept blocks).

The softmax is computed in two passes (all logits, then the maximum, then the
weighted sum). Keys are visited in chunks of ``chunk`` positions only to bound
memory at 128K keys; the chunking changes no arithmetic order that matters in
float64 at the tolerances used.
"""

import numpy as np

from .bf16 import bf16_bits_to_f64


def attend(q, k_bits, v_bits, keys, scale, chunk=8192):
    """Attention output for every query head.

    q       : [Hq][D] array of float32 (or float64) query values.
    k_bits  : [N][Hkv][D] uint16 bf16 bit patterns of the keys at positions 0..N-1.
    v_bits  : [N][Hkv][D] uint16 bf16 bit patterns of the values.
    keys    : 1-D integer array, the positions in S (each position once).
    scale   : softmax scale (1/sqrt(D) by default in the callers).
    returns : [Hq][D] float64.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.int64)
    Hq, D = q.shape
    Hkv = k_bits.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if keys.size == 0:
        raise ValueError("empty key set")
    G = Hq // Hkv
    qg = q.reshape(Hkv, G, D)  # head h = g*G + i uses KV head g

    # pass 1: logits z[j, h]
    z = np.empty((keys.size, Hq), dtype=np.float64)
    for c0 in range(0, keys.size, chunk):
        idx = keys[c0:c0 + chunk]
        K = bf16_bits_to_f64(k_bits[idx])  # [c][Hkv][D]
        for g in range(Hkv):
            z[c0:c0 + idx.size, g * G:(g + 1) * G] = scale * (K[:, g, :] @ qg[g].T)
    m = z.max(axis=0)
    w = np.exp(z - m)
    denom = w.sum(axis=0)

    # pass 2: weighted sum of values
    out = np.zeros((Hq, D), dtype=np.float64)
    for c0 in range(0, keys.size, chunk):
        idx = keys[c0:c0 + chunk]
        V = bf16_bits_to_f64(v_bits[idx])
        for g in range(Hkv):
            out[g * G:(g + 1) * G] += w[c0:c0 + idx.size, g * G:(g + 1) * G].T @ V[:, g, :]
    return out / denom[:, None]


def default_scale(head_dim):
    """1/sqrt(D): the usual scaled-dot-product factor (the pages state none)."""
    return 1.0 / np.sqrt(float(head_dim))
