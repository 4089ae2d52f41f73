"""GPU parity of the weight-bearing ODA step: a 3-layer Qwen3-family decoder
with random weights, history beyond the Local view, the recall head on the real Local
hidden state, the gated recall pass and the select, against the fp64 decoder oracle."""

import pytest

from synth.decoder import decoder_small
from tests.helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("fuse_qk", [True, False])
def test_decoder_oda_steps(fuse_qk):
    # fuse_qk: the per-head q/k finish inside the decode launches (the model's default),
    # else as a launch of its own
    from tests.harness import DecoderRun
    wl = decoder_small()
    rep = DecoderRun(wl, fuse_qk=fuse_qk).run()
    assert rep.decisions == wl.steps and 0 < rep.recalls < wl.steps
    print("decoder_small fuse_qk=%s: recalls %d/%d, max-abs %.2e, row-rel %.2e, commit bf16 mismatches %.4f"
          % (fuse_qk, rep.recalls, wl.steps, rep.max_abs, rep.max_row_rel, rep.commit_mismatch_frac))


def test_decoder_oda_steps_hybrid():
    from tests.harness import DecoderRun
    wl = decoder_small(steps=8)
    rep = DecoderRun(wl, local_only=[1]).run()
    assert rep.decisions == 8
    print("decoder_small hybrid: recalls %d/8, max-abs %.2e" % (rep.recalls, rep.max_abs))


def test_qkv_rope_two_positions():
    """The q/k/v projection with its per-head finish (q/k RMS norm, rotation, bf16 k/v),
    twice in a row on one scratch at a small and a large position, against the fp64
    building blocks of the decoder oracle."""
    import numpy as np
    import torch
    from oracle import decoder as od
    from sparse_kv_recall_amd import ops
    from tests.helpers import bits_to_bf16_tensor
    Hq, Hkv, hidden, eps, base = 16, 8, 2048, 1e-6, 1.0e6
    heads = Hq + 2 * Hkv
    g = np.random.default_rng(77)
    W = (g.standard_normal((heads * 128, hidden)) * 0.02).astype(np.float32)
    Wb = torch.as_tensor(W).to(torch.bfloat16)
    Wd = Wb.float().numpy().astype(np.float64)  # the bf16 weights, widened exactly
    gains = [torch.as_tensor(1.0 + 0.1 * g.standard_normal(n)).to(torch.bfloat16) for n in (hidden, 128, 128)]
    gd = [t.float().numpy().astype(np.float64) for t in gains]
    scratch = torch.zeros(heads * 128, device="cuda")
    q = torch.zeros(Hq * 128, device="cuda")
    k = torch.zeros(Hkv * 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    for call, pos in enumerate((5, 131071)):
        h = g.standard_normal(hidden).astype(np.float32)
        seq = torch.tensor([pos + 1], dtype=torch.int32, device="cuda")
        ops.qkv_rope(Wb.cuda(), torch.as_tensor(h, device="cuda"), gains[0].cuda(), gains[1].cuda(), gains[2].cuda(),
                     Hq, Hkv, seq, scratch, q, k, v, eps=eps, rope_base=base)
        torch.cuda.synchronize()
        raw = Wd @ od.rms_norm(h.astype(np.float64), gd[0], eps)
        heads_ref = raw.reshape(heads, 128)
        q_ref = od.rope(od.rms_norm(heads_ref[:Hq], gd[1], eps), pos, base)
        k_ref = od.rope(od.rms_norm(heads_ref[Hq:Hq + Hkv], gd[2], eps), pos, base)
        v_ref = heads_ref[Hq + Hkv:]
        qg = q.cpu().numpy().reshape(Hq, 128)
        assert np.max(np.abs(qg - q_ref)) <= 1e-3 * max(1.0, np.max(np.abs(q_ref))), call
        for got, ref in ((k, k_ref), (v, v_ref)):
            gt = got.float().cpu().numpy().reshape(-1, 128)
            # bf16 outputs: within one bf16 unit (2^-8 relative) of the fp64 value
            assert np.all(np.abs(gt - ref) <= np.abs(ref) * 2.0 ** -7 + 1e-6), call


@pytest.mark.parametrize("view,G,n,Hkv", [("local", 2, 131072, 2), ("full", 4, 2999, 2), ("local", 8, 6, 2),
                                          ("full", 1, 40, 2), ("full", 2, 1, 2), ("local", 4, 17, 2),
                                          ("full", 4, 3001, 3), ("local", 1, 2100, 16)])
def test_decode_from_projection(view, G, n, Hkv):
    """The Local / Full views from a raw q/k/v projection (per-head q/k RMSNorm and the
    rotation at n - 1 applied inside the decode launch) against the fp64 layer pieces of
    the decoder oracle: the committed v bit for bit, the committed k within one bf16 unit
    of the rounded fp64 key, and the output within the hi+lo error bound of fp64
    attention of the fp64 q over the history with the committed key."""
    import numpy as np
    import torch
    from oracle import attention, keysets
    from oracle import decoder as od
    from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits
    from sparse_kv_recall_amd import ops
    from synth import rng
    from tests.helpers import SCALE, bf16_tensor_to_bits, bits_to_bf16_tensor, check_tight, rand_bits
    eps, base = 1e-6, 1.0e6
    Hq = G * Hkv
    g = np.random.default_rng(100 * G + n % 997)
    mb = -(-n // 16)
    hk = rand_bits(rng.mix_key(911, G, Hkv, 1), n, Hkv)
    hv = rand_bits(rng.mix_key(911, G, Hkv, 2), n, Hkv)
    seq = torch.tensor([n], dtype=torch.int32, device="cuda")
    bt = torch.arange(mb, dtype=torch.int32, device="cuda")[None]
    cache = ops.PagedKVCache(mb, 1, Hq, Hkv, mb, block_tables=bt, seq_lens=seq)
    if n > 1:
        ops.kv_write(cache, 0, 0, bits_to_bf16_tensor(hk[:n - 1]), bits_to_bf16_tensor(hv[:n - 1]))
    raw = (g.standard_normal((Hq + 2 * Hkv, 128)) * 0.7 + 0.1).astype(np.float32)
    gains = [torch.as_tensor(1.0 + 0.2 * g.standard_normal(128)).to(torch.bfloat16) for _ in range(2)]
    gq, gk = (t.float().numpy().astype(np.float64) for t in gains)
    fn = ops.oda_decode_local_qkv if view == "local" else ops.oda_decode_full_qkv
    out = fn(torch.as_tensor(raw).cuda(), gains[0].cuda(), gains[1].cuda(), cache, eps=eps, rope_base=base)
    torch.cuda.synchronize()
    kc, vc = ops.kv_read(cache, 0, n - 1, 1)
    kb, vb = bf16_tensor_to_bits(kc)[0], bf16_tensor_to_bits(vc)[0]
    raw64 = raw.astype(np.float64)
    q = od.rope(od.rms_norm(raw64[:Hq], gq, eps), n - 1, base)
    k = od.rope(od.rms_norm(raw64[Hq:Hq + Hkv], gk, eps), n - 1, base)
    assert np.array_equal(vb, f64_to_bf16_bits(raw64[Hq + Hkv:]))
    kr = f64_to_bf16_bits(k)
    a, b = bf16_bits_to_f64(kb), bf16_bits_to_f64(kr)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-30)
    assert (kb != kr).mean() < 0.05, (kb != kr).mean()
    hk[n - 1], hv[n - 1] = kb, vb
    keys = keysets.local_keys(n) if view == "local" else keysets.full_keys(n)
    ref = attention.attend(q, hk, hv, keys, SCALE)
    check_tight(out[0].cpu().numpy(), ref, q, hk, hv, keys, SCALE, what="%s from projection G=%d Hkv=%d n=%d" % (view, G, Hkv, n))


@pytest.mark.parametrize("view", ["local", "full"])
def test_decode_from_projection_batch(view):
    """The batch (workgroup-planned) instances of the views from a raw projection: three
    requests of different lengths, each with its own projection rows; with a selector
    that skips the second request (its output rows and its slot stay untouched)."""
    import numpy as np
    import torch
    from oracle import attention, keysets
    from oracle import decoder as od
    from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits
    from sparse_kv_recall_amd import ops
    from synth import rng
    from tests.helpers import SCALE, bf16_tensor_to_bits, bits_to_bf16_tensor, check_tight, rand_bits
    B, Hkv, G, eps, base = 3, 2, 4, 1e-6, 1.0e6
    Hq = G * Hkv
    ns = [5000, 300, 2100]
    g = np.random.default_rng(5)
    mb = max(-(-n // 16) for n in ns)
    seq = torch.tensor(ns, dtype=torch.int32, device="cuda")
    bt = torch.arange(B * mb, dtype=torch.int32, device="cuda").view(B, mb)
    cache = ops.PagedKVCache(B * mb, B, Hq, Hkv, mb, block_tables=bt, seq_lens=seq)
    hist = []
    for b, n in enumerate(ns):
        hk = rand_bits(rng.mix_key(912, b, 1), n, Hkv)
        hv = rand_bits(rng.mix_key(912, b, 2), n, Hkv)
        ops.kv_write(cache, b, 0, bits_to_bf16_tensor(hk[:n - 1]), bits_to_bf16_tensor(hv[:n - 1]))
        hist.append((hk, hv))
    slot_before = [tuple(bf16_tensor_to_bits(t)[0].copy() for t in ops.kv_read(cache, b, ns[b] - 1, 1))
                   for b in range(B)]
    raw = (g.standard_normal((B, Hq + 2 * Hkv, 128)) * 0.7 + 0.1).astype(np.float32)
    gains = [torch.as_tensor(1.0 + 0.2 * g.standard_normal(128)).to(torch.bfloat16) for _ in range(2)]
    gq, gk = (t.float().numpy().astype(np.float64) for t in gains)
    sel = torch.tensor([1, 0, 1], dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, 128), 7.0, device="cuda")
    fn = ops.oda_decode_local_qkv if view == "local" else ops.oda_decode_full_qkv
    fn(torch.as_tensor(raw).cuda(), gains[0].cuda(), gains[1].cuda(), cache, eps=eps, rope_base=base, sel=sel,
       sel_value=1, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for b, n in enumerate(ns):
        kc, vc = ops.kv_read(cache, b, n - 1, 1)
        kb, vb = bf16_tensor_to_bits(kc)[0], bf16_tensor_to_bits(vc)[0]
        if b == 1:  # not selected: nothing written
            assert np.all(got[b] == 7.0)
            assert np.array_equal(kb, slot_before[b][0]) and np.array_equal(vb, slot_before[b][1])
            continue
        r64 = raw[b].astype(np.float64)
        q = od.rope(od.rms_norm(r64[:Hq], gq, eps), n - 1, base)
        k = od.rope(od.rms_norm(r64[Hq:Hq + Hkv], gk, eps), n - 1, base)
        assert np.array_equal(vb, f64_to_bf16_bits(r64[Hq + Hkv:])), b
        kr = f64_to_bf16_bits(k)
        a, c = bf16_bits_to_f64(kb), bf16_bits_to_f64(kr)
        assert np.all(np.abs(a - c) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(c)) + 1e-30), b
        hk, hv = hist[b]
        hk[n - 1], hv[n - 1] = kb, vb
        keys = keysets.local_keys(n) if view == "local" else keysets.full_keys(n)
        ref = attention.attend(q, hk, hv, keys, SCALE)
        check_tight(got[b], ref, q, hk, hv, keys, SCALE, what="%s from projection b=%d n=%d" % (view, b, n))


def test_host_routed_model_equals_one_graph():
    """The weight-bearing step with the recall pass routed on the host (two graphs split at
    the recall head's gate, the select in both branches) against the one-graph step: the
    same launches in the same order, so every step's selected and Local final hidden
    states and every committed slot are bit-identical, and the recall graph runs exactly
    on the steps whose gate is set."""
    import numpy as np
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.model import DecoderShape, ODADecoder
    from sparse_kv_recall_amd.stack import HostRoutedStep, capture_graph
    wl = decoder_small(steps=12)
    runs = []
    for host in (False, True):
        mb = wl.max_blocks
        bt = torch.arange(mb, dtype=torch.int32, device="cuda")[None]
        seq = torch.full((1,), wl.H0, dtype=torch.int32, device="cuda")
        caches = [ops.PagedKVCache(mb, 1, wl.q_heads, wl.kv_heads, mb, block_tables=bt, seq_lens=seq)
                  for _ in range(wl.layers)]
        for l, c in enumerate(caches):
            k = wl.hist_bits("k", l, 0, wl.H0)
            v = wl.hist_bits("v", l, 0, wl.H0)
            ops.kv_write(c, 0, 0, torch.as_tensor(k.view(np.int16), device="cuda").view(torch.bfloat16),
                         torch.as_tensor(v.view(np.int16), device="cuda").view(torch.bfloat16))
        shape = DecoderShape(wl.layers, wl.hidden, wl.q_heads, wl.kv_heads, wl.intermediate, wl.vocab,
                             wl.recall_hidden, wl.eps, wl.rope_base)
        m = ODADecoder(shape, wl.device_weights(), caches, wl.sinks, wl.window)
        tokens = torch.as_tensor(wl.tokens.astype(np.int64), device="cuda")
        t_idx = torch.zeros(1, dtype=torch.int64, device="cuda")

        def feed():
            m.token.copy_(torch.index_select(tokens, 0, t_idx))
            seq.add_(1)
            t_idx.add_(1)

        def first():
            feed()
            m.local_pass()
            m.recall_gate(wl.theta)

        def select():
            ops.select(m.gate, m.final_full, m.h_local_final, m.h_prev)

        def recall():
            m.recall_pass(gated=True)
            select()

        def one_graph():
            first()
            recall()

        step = HostRoutedStep(first, recall, m.gate, skip=select) if host else capture_graph(one_graph)
        states, ran = [], []
        for _ in range(wl.steps):
            r = step.replay()
            torch.cuda.synchronize()
            states.append((m.h_prev.clone(), m.h_local_final.clone(), int(m.gate[0].item())))
            ran.append(r)
        slots = [ops.kv_read(c, 0, wl.H0, wl.steps) for c in caches]
        runs.append((states, ran, slots))
    (s0, _, k0), (s1, ran1, k1) = runs
    gates = [g for _, _, g in s0]
    assert 0 < sum(gates) < wl.steps
    for t in range(wl.steps):
        assert torch.equal(s0[t][0], s1[t][0]) and torch.equal(s0[t][1], s1[t][1]), t
        assert s0[t][2] == s1[t][2] and ran1[t] == bool(s1[t][2]), t
    for (ka, va), (kb, vb) in zip(k0, k1):
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16))
        assert torch.equal(va.view(torch.int16), vb.view(torch.int16))
