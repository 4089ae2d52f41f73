"""Shared test plumbing: building paged caches from host arrays, tolerance checks."""

import math

import numpy as np
import pytest
import torch

from synth import rng

SCALE = 1.0 / math.sqrt(128.0)
NAN_BF16 = 0x7FC0

# Tolerance for attention outputs (fp32 GPU vs fp64 oracle): max-abs 2e-3 over all
# elements AND, per (request, head) row, max|diff| / max|ref| <= 1e-2.
ABS_TOL = 2e-3
ROW_REL_TOL = 1e-2


def gpu_available():
    try:
        return torch.cuda.is_available()
    except Exception:
        return False


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs a GPU")


def bits_to_bf16_tensor(bits, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_tensor_to_bits(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def rand_bits(key, count, Hkv):
    return rng.normal_bf16(key, 0, count * Hkv * 128, rng.unit_scale()).reshape(count, Hkv, 128)


def rand_f32(key, shape, sigma=1.0):
    n = int(np.prod(shape))
    return rng.normal_f32(key, 0, n, rng.unit_scale(sigma)).reshape(shape)


def check_close(got, ref, abs_tol=ABS_TOL, row_rel_tol=ROW_REL_TOL, what=""):
    """got, ref: [..., 128] arrays. Returns (max_abs, max_row_rel)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite output %s" % what
    diff = np.abs(got - ref)
    max_abs = float(diff.max()) if diff.size else 0.0
    rows_d = diff.reshape(-1, diff.shape[-1]).max(axis=1)
    rows_r = np.abs(ref).reshape(-1, ref.shape[-1]).max(axis=1)
    row_rel = float((rows_d / np.maximum(rows_r, 1e-30)).max()) if rows_d.size else 0.0
    assert max_abs <= abs_tol, "max-abs %.3e > %.1e %s" % (max_abs, abs_tol, what)
    assert row_rel <= row_rel_tol, "row-rel %.3e > %.1e %s" % (row_rel, row_rel_tol, what)
    return max_abs, row_rel


# ---- kernel error model (for the tight checks) --------------------------------
# The decode kernels take q' = q * scale * log2(e) in fp32 and split it into bf16
# high + low parts; K and V are exact bf16; the logits (base 2) accumulate in fp32 on
# the matrix cores; the softmax weights p enter the PV product as bf16 high + low
# parts too, while their sum l stays fp32. Two round-to-nearest roundings to 8
# significant bits leave a residual of at most 2^-16 of the value, so:
#   logit error     |dt_j| <= (2^-16 + 2^-20) * A_j,  A_j = sum_d |q'_d| |k_jd|
#                   (2^-20 covers the fp32 accumulation of the 8 chained products)
#   weight error    eps_j  <= ln 2 * |dt_j| + 2^-22   (exp2 of the hardware)
#   normalised      |do_d| <= 2 E / (1 - E) * sum_j p_j |v_jd - o_d|,  E = max_j eps_j
#   PV split        |do_d| <= 2^-16 * sum_j p_j |v_jd|
# plus the fp32 sums over tiles, waves and splits, taken as a random walk of unit
# roundoffs, 2^-22 * sqrt(tiles + 1) * max|v|, and one rounding of the output. The
# bound is per (request, head) row and is computed from the inputs themselves.
LOG2E = 1.4426950408889634


def hilo_bound(q, k_bits, v_bits, keys, scale):
    """Per-row bound [Hq] of |GPU - fp64| for attention over `keys` (see above)."""
    from oracle.bf16 import bf16_bits_to_f64
    q = np.asarray(q, np.float64)
    keys = np.asarray(keys, np.int64)
    Hq = q.shape[0]
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    tiles = -(-int(keys.size) // 16)
    out = np.zeros(Hq)
    for g in range(Hkv):
        K = bf16_bits_to_f64(k_bits[keys, g])  # [nk][D]
        V = bf16_bits_to_f64(v_bits[keys, g])
        vmax = float(np.abs(V).max())
        for i in range(G):
            h = g * G + i
            qp = q[h] * scale * LOG2E
            A = np.abs(K) @ np.abs(qp)
            E = float(math.log(2.0) * (2.0 ** -16 + 2.0 ** -20) * A.max() + 2.0 ** -22)
            z = scale * (K @ q[h])
            w = np.exp(z - z.max())
            p = w / w.sum()
            o = p @ V
            s1 = p @ np.abs(V - o)
            s2 = p @ np.abs(V)
            row = 2 * E / (1 - E) * s1 + 2.0 ** -16 * s2
            out[h] = float(row.max()) + 2.0 ** -22 * math.sqrt(tiles + 1) * vmax + 2.0 ** -24 * float(np.abs(o).max())
    return out


def check_tight(got, ref, q, k_bits, v_bits, keys, scale=SCALE, what=""):
    """Every (head) row of `got` [Hq][D] within the error model's bound of the fp64
    reference `ref`; also the tolerance reading of the scope (check_close). Returns the
    largest observed |error| / bound over the rows."""
    check_close(got, ref, what=what)
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = hilo_bound(q, k_bits, v_bits, keys, scale)
    err = np.abs(got - ref).max(axis=1)
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, "rows %s: error %s above the hi+lo bound %s %s" % (
        bad[:4].tolist(), err[bad[:4]].tolist(), bound[bad[:4]].tolist(), what)
    return float((err / bound).max())


class HostCache:
    """Logical per-request K/V (bf16 bits) mirrored into a GPU paged cache."""

    def __init__(self, Hq, Hkv, ns, seed=0, permute=True, poison=True, spare_blocks=3, max_blocks=None,
                 device="cuda"):
        from sparse_kv_recall_amd import ops

        self.Hq, self.Hkv, self.ns = Hq, Hkv, list(ns)
        B = len(ns)
        nb = [(n + 15) // 16 for n in ns]
        self.max_blocks = max_blocks or max(nb)
        total = sum(self.max_blocks for _ in ns) + spare_blocks
        g = np.random.default_rng(1000 + seed)
        phys = g.permutation(total) if permute else np.arange(total)
        bt = np.zeros((B, self.max_blocks), np.int32)
        for b in range(B):
            bt[b] = phys[b * self.max_blocks:(b + 1) * self.max_blocks]
        self.bt = bt
        self.kv = ops.PagedKVCache(total, B, Hq, Hkv, self.max_blocks, device=device,
                                   block_tables=torch.as_tensor(bt, device=device),
                                   seq_lens=torch.as_tensor(np.asarray(ns, np.int32), device=device))
        if poison:
            self.kv.k_pool.view(torch.int16).fill_(NAN_BF16)
            self.kv.v_pool.view(torch.int16).fill_(NAN_BF16)
        else:
            self.kv.k_pool.zero_()
            self.kv.v_pool.zero_()
        self.k = []
        self.v = []
        for b, n in enumerate(ns):
            kb = rand_bits(rng.mix_key(900, seed, 1, b), self.max_blocks * 16, Hkv)
            vb = rand_bits(rng.mix_key(900, seed, 2, b), self.max_blocks * 16, Hkv)
            self.k.append(kb)
            self.v.append(vb)
            if n > 0:
                ops.kv_write(self.kv, b, 0, bits_to_bf16_tensor(kb[:n], device),
                             bits_to_bf16_tensor(vb[:n], device))

    def set_lens(self, ns):
        self.ns = list(ns)
        self.kv.seq_lens.copy_(torch.as_tensor(np.asarray(ns, np.int32)))
