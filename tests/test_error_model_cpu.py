"""CPU check of the error model behind the tight GPU checks (tests/helpers.py hilo_bound).

An emulation of the decode kernels' arithmetic in numpy float32 -- q' = q * scale *
log2(e) split into bf16 high + low parts, base-2 logits accumulated in float32,
exp2 in float32, the weights split into bf16 high + low parts for the PV product and
summed unsplit for the denominator -- must stay within the bound of the fp64 oracle
on every row, over small and large key sets, peaky queries and a single key. A model
that left out a term the kernel has (the weights' split, say) fails here; and the
emulation must be distinguishable from exact arithmetic, or the check tests nothing.
"""

import numpy as np
import pytest

from oracle import attention, keysets
from oracle.bf16 import bf16_bits_to_f64
from synth import rng
from tests.helpers import LOG2E, SCALE, hilo_bound, rand_bits, rand_f32


def _bf16(x):
    from oracle.bf16 import f64_to_bf16_bits
    return bf16_bits_to_f64(f64_to_bf16_bits(np.asarray(x, np.float64))).astype(np.float32)


def emulate(q, k_bits, v_bits, keys, scale):
    Hq = q.shape[0]
    Hkv = k_bits.shape[1]
    G = Hq // Hkv
    out = np.zeros((Hq, 128))
    for g in range(Hkv):
        K = bf16_bits_to_f64(k_bits[keys, g]).astype(np.float32)
        V = bf16_bits_to_f64(v_bits[keys, g]).astype(np.float32)
        for i in range(G):
            h = g * G + i
            qp = np.asarray(q[h], np.float32) * np.float32(scale * LOG2E)
            hi = _bf16(qp)
            lo = _bf16(qp - hi)
            t = (K @ hi + K @ lo).astype(np.float32)
            p = np.exp2(t - t.max()).astype(np.float32)
            ph = _bf16(p)
            pl = _bf16(p - ph)
            acc = (ph @ V + pl @ V).astype(np.float32)
            out[h] = acc / np.float32(p.sum(dtype=np.float32))
    return out


@pytest.mark.parametrize("n,sigma,seed", [(1, 1.0, 0), (4, 1.0, 1), (37, 1.0, 2), (2052, 1.0, 3),
                                          (9000, 1.0, 4), (300, 8.0, 5)])
def test_emulated_kernel_arithmetic_within_bound(n, sigma, seed):
    Hq, Hkv = 8, 2
    k = rand_bits(rng.mix_key(990, seed, 1), n, Hkv)
    v = rand_bits(rng.mix_key(990, seed, 2), n, Hkv)
    q = rand_f32(rng.mix_key(990, seed, 3), (Hq, 128), sigma)
    keys = keysets.full_keys(n)
    ref = attention.attend(q, k, v, keys, SCALE)
    got = emulate(q, k, v, keys, SCALE)
    bound = hilo_bound(q, k, v, keys, SCALE)
    err = np.abs(got - ref).max(axis=1)
    assert (err <= bound).all(), (err, bound)
    if n > 1:
        assert err.max() > 0.0  # the emulation does round


def test_bound_fails_without_the_low_parts():
    # dropping the low bf16 parts (one rounding to 8 bits instead of two) breaks the
    # bound on some row: the bound is tight enough to see the split
    n, Hq, Hkv = 64, 8, 2
    k = rand_bits(rng.mix_key(991, 1), n, Hkv)
    v = rand_bits(rng.mix_key(991, 2), n, Hkv)
    q = rand_f32(rng.mix_key(991, 3), (Hq, 128), 2.0)
    keys = keysets.full_keys(n)
    ref = attention.attend(q, k, v, keys, SCALE)
    bound = hilo_bound(q, k, v, keys, SCALE)
    out = np.zeros((Hq, 128))
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = bf16_bits_to_f64(k[keys, g]).astype(np.float32)
        V = bf16_bits_to_f64(v[keys, g]).astype(np.float32)
        t = K @ _bf16(np.asarray(q[h], np.float32) * np.float32(SCALE * LOG2E))
        p = np.exp2(t - t.max()).astype(np.float32)
        out[h] = (_bf16(p) @ V) / p.sum(dtype=np.float32)
    err = np.abs(out - ref).max(axis=1)
    assert (err > bound).any(), (err, bound)
