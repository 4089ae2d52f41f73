"""GPU parity of whole decode steps on the five seeded workloads, at their full sizes,
in the launch configuration the benchmark times (a captured HIP graph per step).

Outputs are checked on sampled layers / requests / steps that the fp64 oracle can
compute one by one; decisions, gathered block lists and commits are checked on every
step. See tests/harness.py for what each run compares.
"""

import numpy as np
import pytest

from synth import workloads
from tests.helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_oda_small_every_step():
    from tests.harness import OdaStackRun
    wl = workloads.oda_small()
    rep = OdaStackRun(wl, check_layers=[0]).run(check_feed_steps=(0, 5))
    assert rep.decisions == 64 and rep.checked_outputs == 64 + rep.recalls
    print("oda_small: recalls %d/64, max-abs %.2e, row-rel %.2e" % (rep.recalls, rep.max_abs, rep.max_row_rel))


def test_oda_stack16k_recall_head():
    from tests.harness import OdaStackRun
    wl = workloads.oda_stack16k()
    rep = OdaStackRun(wl, check_layers=[0, 1, 27]).run()
    assert rep.decisions == 256
    assert 0 < rep.recalls < 256
    print("oda_stack16k: recalls %d/256 (%d in the 1e-4 band), max-abs %.2e, row-rel %.2e"
          % (rep.recalls, rep.decisions_in_band, rep.max_abs, rep.max_row_rel))


@pytest.mark.slow
def test_oda_stack128k_metric_workload():
    # every decision; Local outputs of six seeded layers on every step; Full outputs of
    # those layers on eight seeded recall steps and the last, and on every other recall
    # step the four query heads of one seeded KV head of one of them; committed slots of
    # all 36 layers on every step (the selected pass's candidates, bit for bit)
    from tests.harness import OdaStackRun
    wl = workloads.oda_stack128k()
    g = np.random.default_rng(3)
    layers = sorted(set([0, 35] + [int(x) for x in g.choice(np.arange(1, 35), size=4, replace=False)]))
    recall_steps = np.flatnonzero(wl.sched_scores[:, 0] > 0)
    sample = set(int(x) for x in g.choice(recall_steps, size=8, replace=False))
    sample.add(int(recall_steps[-1]))
    rep = OdaStackRun(wl, check_layers=layers).run(full_check_steps=sample, commit_all_layers=True,
                                                   full_sample=np.random.default_rng(4))
    assert rep.decisions == 1024 and rep.recalls == 128 and rep.commit_layers == 36
    assert rep.checked_outputs == 1024 * len(layers) + len(sample) * len(layers) + (128 - len(sample))
    print("oda_stack128k: local checked every step on layers %s; full checked at steps %s (one sampled KV head "
          "on the other recall steps); commits of all 36 layers; max-abs %.2e, row-rel %.2e"
          % (layers, sorted(sample), rep.max_abs, rep.max_row_rel))


@pytest.mark.parametrize("in_kernel_rewrite", [False, True])
def test_da_32k_every_step(in_kernel_rewrite):
    from tests.harness import DaRun
    wl = workloads.da_32k()
    rep = DaRun(wl, in_kernel_rewrite=in_kernel_rewrite).run()
    assert rep.checked_outputs == 512
    print("da_32k (rewrite in kernel: %s): max-abs %.2e, row-rel %.2e" % (in_kernel_rewrite, rep.max_abs,
                                                                         rep.max_row_rel))


@pytest.mark.slow
@pytest.mark.parametrize("one_launch", [True, False])
def test_ragged32_sampled_requests(one_launch):
    # the three views in one launch (oda_decode_views), and one selector launch per view;
    # every request's view decision on every step, the outputs of six requests on every
    # eighth step, and every request's committed slots on every step
    from tests.harness import RaggedRun
    wl = workloads.ragged32()
    order = np.argsort(wl.H0)
    check = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2])] +
                       [int(x) for x in np.random.default_rng(4).choice(wl.batch, size=3, replace=False)]))
    rep = RaggedRun(wl, check_requests=check, one_launch=one_launch).run(
        check_steps=set(range(0, wl.steps, 8)) | {wl.steps - 1}, commit_all_requests=True)
    assert rep.decisions == wl.batch * wl.steps and rep.commit_layers == wl.batch
    print("ragged32 (one launch: %s): requests %s, full views %d of %d, max-abs %.2e, row-rel %.2e"
          % (one_launch, check, rep.recalls, rep.decisions, rep.max_abs, rep.max_row_rel))


def test_hybrid_local_only_layers():
    # per-layer access control: three of every four layers restricted to the Local range
    from tests.harness import OdaStackRun
    wl = workloads.oda_stack16k(steps=48)
    local_only = [l for l in range(wl.layers) if l % 4 != 3]
    rep = OdaStackRun(wl, check_layers=[0, 3, 26, 27], local_only=local_only).run()
    assert rep.decisions == 48 and rep.recalls > 0
    print("hybrid: recalls %d/48, max-abs %.2e, row-rel %.2e" % (rep.recalls, rep.max_abs, rep.max_row_rel))


def test_all_layers_local_only_equals_local():
    # with every layer local-only and the recall pass fed what the Local pass saw, the
    # step's output is the Local output bit for bit, and so are the commits
    from tests.harness import OdaStackRun
    wl = workloads.oda_stack16k(steps=24, layers=4)
    rep = OdaStackRun(wl, check_layers=[0, 1, 2, 3], local_only=range(4), same_candidates=True).run()
    assert rep.recalls > 0
    print("all local-only: recalls %d/24, max-abs %.2e" % (rep.recalls, rep.max_abs))


@pytest.mark.parametrize("in_kernel_rewrite", [False, True])
def test_da_tag_stream_every_step(in_kernel_rewrite):
    # declarations parsed on the device from a token stream (mode tags, named segments)
    from tests.harness import DaTagsRun
    wl = workloads.da_tags_32k()
    rep = DaTagsRun(wl, in_kernel_rewrite=in_kernel_rewrite).run()
    assert rep.checked_outputs == 512 and rep.recalls > 0
    print("da_tags_32k: focus steps %d/512, max-abs %.2e, row-rel %.2e" % (rep.recalls, rep.max_abs, rep.max_row_rel))


def test_oda_stack16k_host_routed():
    # the step as two graphs with the recall branch taken on the host: the recall-head
    # workload checked like the one-graph step, and the recall graph replayed only on the
    # steps whose device gate is set
    from tests.harness import OdaStackRun
    wl = workloads.oda_stack16k(steps=48)
    rep = OdaStackRun(wl, check_layers=[0, 13, 27], host_routed=True).run(commit_all_layers=True)
    assert rep.decisions == 48 and 0 < rep.recalls < 48
    print("host-routed 16K: recalls %d/48, max-abs %.2e, row-rel %.2e" % (rep.recalls, rep.max_abs, rep.max_row_rel))


def test_host_routed_equals_one_graph_step():
    # same launches, same order: per-step outputs and the committed slots are bit-identical
    import torch
    from sparse_kv_recall_amd import ops
    from tests.harness import OdaStackRun
    wl = workloads.oda_stack16k(steps=24, layers=4)
    runs = [OdaStackRun(wl, check_layers=[], host_routed=h) for h in (False, True)]
    outs = [[], []]
    for i, r in enumerate(runs):
        for t in range(wl.steps):
            r.graph.replay()
            torch.cuda.synchronize()
            outs[i].append((r.stack.out.clone(), r.stack.out_full.clone() if r.stack.gate[0].item() else None))
    recalls = 0
    for t in range(wl.steps):
        (a, af), (b, bf) = outs[0][t], outs[1][t]
        assert torch.equal(a, b), t
        assert (af is None) == (bf is None), t
        if af is not None:
            assert torch.equal(af, bf), t
            recalls += 1
    assert 0 < recalls < wl.steps
    H0 = int(wl.H0[0])
    for l in range(wl.layers):
        ka, va = ops.kv_read(runs[0].stack.caches[l], 0, H0, wl.steps)
        kb, vb = ops.kv_read(runs[1].stack.caches[l], 0, H0, wl.steps)
        assert torch.equal(ka.view(torch.int16), kb.view(torch.int16)) and torch.equal(va.view(torch.int16),
                                                                                        vb.view(torch.int16)), l
