"""GPU parity of the weight-bearing ODA step: a 3-layer Qwen3-family decoder
with random weights, history beyond the Local view, the recall head on the real Local
hidden state, the gated recall pass and the select, against the fp64 decoder oracle."""

import pytest

from synth.decoder import decoder_small
from tests.helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_decoder_oda_steps():
    from tests.harness import DecoderRun
    wl = decoder_small()
    rep = DecoderRun(wl).run()
    assert rep.decisions == wl.steps and 0 < rep.recalls < wl.steps
    print("decoder_small: recalls %d/%d, max-abs %.2e, row-rel %.2e, commit bf16 mismatches %.4f"
          % (rep.recalls, wl.steps, rep.max_abs, rep.max_row_rel, rep.commit_mismatch_frac))


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
