"""GPU parity of the weight-bearing ODA step (NEXT-2): a 3-layer Qwen3-family decoder
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
