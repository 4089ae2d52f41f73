"""Pins of the weight-bearing decoder's layer (oracle/decoder.py Decoder.layer) by a second,
independent formulation: scalar Python loops over one Qwen3-family decoder layer written
from its published description (pre-norm RMSNorm; q, k, v projections; RMSNorm of each
q and k head; rotate-half rotary embedding at the current position n - 1 on q and on the
key that is committed; attention over the view; output projection and residual; RMSNorm;
SiLU of the gate half times the up half; down projection and residual).

The comparison fails for the plausible slips of such a layer -- the head norm after the
rotation, the rotation at position n instead of n - 1, SiLU on the up half -- as the
mutated formulations below show; and the committed key's rotation angle is read back
from its bits. The pages give no layer of their own (parity of the layer structure
itself rests on the model family's published layer)."""

import math

import numpy as np
import pytest

import oracle
from oracle import decoder
from tests.test_oracle_pins import _hist, _tiny_decoder

TOL = 1e-12


def _bf16(x):
    """Round to 8 significant bits, ties to even (Python's round is half-to-even)."""
    if x == 0.0:
        return 0.0
    m, e = math.frexp(x)
    return math.ldexp(round(math.ldexp(m, 8)), e - 8)


def _rms(v, g, eps):
    r = math.sqrt(sum(x * x for x in v) / len(v) + eps)
    return [v[i] / r * g[i] for i in range(len(v))]


def _gemv(W, x):
    return [sum(W[r][c] * x[c] for c in range(len(x))) for r in range(len(W))]


def _rope(v, pos, base):
    D = len(v)
    half = D // 2
    out = [0.0] * D
    for i in range(half):
        a = pos * base ** (-2.0 * i / D)
        c, s = math.cos(a), math.sin(a)
        out[i] = v[i] * c - v[i + half] * s
        out[i + half] = v[i + half] * c + v[i] * s
    return out


def scalar_layer(w, s, l, h, hist_k, hist_v, n, keys, scale, mutate=None):
    """One layer by scalar loops. hist_k / hist_v: float lists [pos][g][d] of the history
    (position n-1 is replaced by this layer's committed key / value). Returns (h, k_commit,
    v_commit, k_normed) with k_commit the bf16 values written at n-1 and k_normed the key
    heads after their RMSNorm, before the rotation."""
    D, Hq, Hkv, eps = s.head_dim, s.q_heads, s.kv_heads, s.eps
    W = lambda name: w["%s.%d" % (name, l)]
    x = _rms(list(h), W("g_attn"), eps)
    qkv = _gemv(W("qkv"), x)
    q = [qkv[i * D:(i + 1) * D] for i in range(Hq)]
    k = [qkv[(Hq + g) * D:(Hq + g + 1) * D] for g in range(Hkv)]
    v = [qkv[(Hq + Hkv + g) * D:(Hq + Hkv + g + 1) * D] for g in range(Hkv)]
    pos = n if mutate == "position" else n - 1
    if mutate == "rope_before_norm":
        q = [_rms(_rope(r, pos, s.rope_base), W("g_q"), eps) for r in q]
        k_normed = [_rms(r, W("g_k"), eps) for r in k]
        k = [_rms(_rope(r, pos, s.rope_base), W("g_k"), eps) for r in k]
    else:
        q = [_rope(_rms(r, W("g_q"), eps), pos, s.rope_base) for r in q]
        k_normed = [_rms(r, W("g_k"), eps) for r in k]
        k = [_rope(r, pos, s.rope_base) for r in k_normed]
    kc = [[_bf16(x) for x in r] for r in k]
    vc = [[_bf16(x) for x in r] for r in v]
    G = Hq // Hkv
    o = []
    for hh in range(Hq):
        g = hh // G
        kk = lambda j: kc[g] if j == n - 1 else hist_k[j][g]
        vv = lambda j: vc[g] if j == n - 1 else hist_v[j][g]
        z = [scale * sum(q[hh][d] * kk(j)[d] for d in range(D)) for j in keys]
        m = max(z)
        e = [math.exp(t - m) for t in z]
        tot = sum(e)
        o += [sum(e[i] * vv(j)[d] for i, j in enumerate(keys)) / tot for d in range(D)]
    h = [h[i] + t for i, t in enumerate(_gemv(W("o"), o))]
    x = _rms(h, W("g_mlp"), eps)
    gu = _gemv(W("gu"), x)
    I = s.intermediate
    gate, up = (gu[I:], gu[:I]) if mutate == "silu_on_up" else (gu[:I], gu[I:])
    a = [gate[i] / (1.0 + math.exp(-gate[i])) * up[i] for i in range(I)]
    h = [h[i] + t for i, t in enumerate(_gemv(W("down"), a))]
    return h, kc, vc, k_normed


def _setup(seed, n):
    dec = _tiny_decoder(seed)
    hist = _hist(dec, n, seed + 1)
    w = {k: v.tolist() for k, v in dec.w.items()}
    h0 = dec.w["emb"][9] * 0.7 + 0.1
    hk = oracle.bf16_bits_to_f64(hist[0][0]).tolist()
    hv = oracle.bf16_bits_to_f64(hist[0][1]).tolist()
    return dec, hist, w, h0, hk, hv


@pytest.mark.parametrize("full", [False, True])
def test_layer_equals_scalar_formulation(full):
    n, window = 300, 64
    dec, hist, w, h0, hk, hv = _setup(21, n)
    keys = list(range(n)) if full else sorted(set(range(4)) | set(range(n - window, n)))
    scale = 1.0 / math.sqrt(128.0)
    ref_h, kc, vc, _ = scalar_layer(w, dec.s, 0, h0.tolist(), hk, hv, n, keys, scale)
    got_h = dec.layer(0, h0.copy(), hist[0][0], hist[0][1], n, full, scale, 4, window)
    assert np.max(np.abs(np.asarray(ref_h) - got_h)) <= TOL * max(1.0, float(np.max(np.abs(got_h))))
    # the slot holds the rotated, normalised key and the value, rounded to bf16
    assert np.array_equal(oracle.bf16_bits_to_f64(hist[0][0][n - 1]), np.asarray(kc))
    assert np.array_equal(oracle.bf16_bits_to_f64(hist[0][1][n - 1]), np.asarray(vc))


@pytest.mark.parametrize("mutate", ["rope_before_norm", "position", "silu_on_up"])
def test_scalar_formulation_sees_the_slips(mutate):
    # each slip moves the layer's output far outside the comparison's tolerance
    n = 300
    dec, hist, w, h0, hk, hv = _setup(22, n)
    keys = list(range(n))
    scale = 1.0 / math.sqrt(128.0)
    got_h = dec.layer(0, h0.copy(), hist[0][0], hist[0][1], n, True, scale, 4, 64)
    bad_h, _, _, _ = scalar_layer(w, dec.s, 0, h0.tolist(), hk, hv, n, keys, scale, mutate=mutate)
    assert np.max(np.abs(np.asarray(bad_h) - got_h)) > 1e6 * TOL


def test_committed_key_carries_the_rotation_of_position_n_minus_1():
    # read the committed key's bits back and recover, pair by pair, the angle by which the
    # normalised key was rotated: (n - 1) * base^(-2i/D) modulo 2 pi for the fast pairs
    n = 300
    dec, hist, w, h0, hk, hv = _setup(23, n)
    scale = 1.0 / math.sqrt(128.0)
    _, _, _, k_normed = scalar_layer(w, dec.s, 0, h0.tolist(), hk, hv, n, list(range(n)), scale)
    dec.layer(0, h0.copy(), hist[0][0], hist[0][1], n, True, scale, 4, 64)
    c = oracle.bf16_bits_to_f64(hist[0][0][n - 1][0])
    u = np.asarray(k_normed[0])
    D, half, base = 128, 64, dec.s.rope_base
    checked = 0
    for i in range(8):
        if math.hypot(u[i], u[i + half]) < 0.3:
            continue  # too short a pair to read an angle from bf16 values
        ang = math.atan2(u[i] * c[i + half] - u[i + half] * c[i], u[i] * c[i] + u[i + half] * c[i + half])
        want = (n - 1) * base ** (-2.0 * i / D)
        diff = (ang - want + math.pi) % (2 * math.pi) - math.pi
        assert abs(diff) < 0.03, (i, ang, want)
        wrong = (ang - n * base ** (-2.0 * i / D) + math.pi) % (2 * math.pi) - math.pi
        assert abs(wrong) > 0.1  # position n would be seen
        checked += 1
    assert checked >= 4
