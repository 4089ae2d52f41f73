#!/usr/bin/env python3
"""Decode-attention throughput of On-Demand Attention at a 128K context, 12.5 % recall.

Workload (synthetic, seeded; stands in for the ODA summary page's 128K-input / 1K-output
vLLM measurement in "Main results"): a 36-layer attention stack with 32 query / 8 KV
heads, head dim 128, bf16 paged KV (block 16) holding 131072 history positions that
grows by one position per decode step, batch 1. Every step runs, per layer, the Local
view (4 sinks + 2048-position window, current token committed), then the on-device
gate, then the gated Full view over the whole history (recomputing the step and
committing the Full candidate) on exactly 128 of the 1024 steps.

One step = one replay of a HIP graph holding: the input feed (synthetic projections:
the step's q / k / v candidates and the length n), the Local view's tile table (its physical
blocks, listed once for all layers), 36 Local launches, the gate, and 36
gated Full launches. Inputs are resident in HBM before timing starts.

Output: one JSON line (metric, tokens/s, ms per step, the roofline of the dominant
kernel -- the Full view at n ~ 132K -- and the fp64 oracle timed on the host cores).
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn tokens/s at 128K ctx, 12.5% recall rate; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
RECALL_PERIOD = 8  # one Full (recall) step in every aligned run of 8 steps: 12.5 %


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def build_stack(wl, device):
    import torch
    from sparse_kv_recall_amd.stack import ODAStack
    from synth import device as sdev
    from synth.workloads import C_KHIST, C_VHIST

    bt = torch.as_tensor(wl.block_tables, device=device)
    seq_lens = torch.zeros(wl.batch, dtype=torch.int32, device=device)
    stack = ODAStack(wl.layers, wl.batch, wl.Hq, wl.Hkv, wl.num_phys_blocks, wl.max_blocks, bt, seq_lens,
                     sinks=wl.sinks, window=wl.window, device=device)
    H0 = int(wl.H0[0])
    from sparse_kv_recall_amd import ops
    stage_k = torch.empty((H0, wl.Hkv, 128), dtype=torch.bfloat16, device=device)
    stage_v = torch.empty_like(stage_k)
    for l in range(wl.layers):
        sdev.fill_normal_(stage_k, wl.key(C_KHIST, l), 0)
        sdev.fill_normal_(stage_v, wl.key(C_VHIST, l), 0)
        ops.kv_write(stack.caches[l], 0, 0, stage_k, stage_v)
    torch.cuda.synchronize()
    del stage_k, stage_v
    return stack


def capture_step(stack, feeder):
    from sparse_kv_recall_amd.stack import capture_graph
    q, k, v = feeder.q, feeder.k, feeder.v

    def step():
        feeder.step()
        stack.local_pass(q[:, 0, :], k[:, 0, :], v[:, 0, :])
        stack.gate_from_scores(feeder.scores, 0.0)
        stack.full_pass(q[:, 1, :], k[:, 1, :], v[:, 1, :], gated=True)

    return capture_graph(step)


def host_routed_rate(stack, feeder, wl, steps, warmup):
    """The metric workload's first `steps` steps again with the recall branch taken on the
    host: graph 1 (feed, Local pass, gate), a 4-byte readback of the gate, and graph 2 (the
    36 gated Full launches) replayed only on recall steps. Same launches and results as the
    one-graph step; the skipped launches cost no graph nodes, each step pays one host round
    trip instead. Weighted 1 : 7 like the metric."""
    import numpy as np
    import torch
    from sparse_kv_recall_amd.stack import HostRoutedStep

    q, k, v = feeder.q, feeder.k, feeder.v

    def first():
        feeder.step()
        stack.local_pass(q[:, 0, :], k[:, 0, :], v[:, 0, :])
        stack.gate_from_scores(feeder.scores, 0.0)

    def recall():
        stack.full_pass(q[:, 1, :], k[:, 1, :], v[:, 1, :], gated=True)

    step = HostRoutedStep(first, recall, stack.gate)
    feeder.set_step(0)
    for _ in range(warmup):
        step.replay()
    feeder.set_step(0)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ran = np.zeros(steps, bool)
    wall0 = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        ran[i] = step.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    rec = wl.sched_scores[:steps, 0] > 0
    assert np.array_equal(ran, rec), "host routing disagrees with the schedule"
    ms_rec, ms_non = float(per_step[rec].mean()), float(per_step[~rec].mean())
    ms = (ms_rec + (RECALL_PERIOD - 1) * ms_non) / RECALL_PERIOD
    del step
    return {"tok_s": round(wl.batch / (ms / 1e3), 2), "ms_per_step": round(ms, 4), "recall_step_ms": round(ms_rec, 4),
            "other_step_ms": round(ms_non, 4), "steps": steps, "recall_steps": int(rec.sum()),
            "wall_ms_per_step": round(wall * 1e3 / steps, 4)}


def roofline_full(stack, feeder, reps):
    """Average duration of the Full-view kernel over all layers at the current n, with HIP
    events on the launching stream; every launch runs (no gate)."""
    import torch
    q, k, v = feeder.q, feeder.k, feeder.v
    stack.full_pass(q[:, 1, :], k[:, 1, :], v[:, 1, :], gated=False)  # warm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        stack.full_pass(q[:, 1, :], k[:, 1, :], v[:, 1, :], gated=False)
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / (reps * stack.layers)


def view_sweep(device, Hq=32, Hkv=8, reps=10, min_bytes=1 << 30):
    """Full and Local views over context lengths at batch 1 and over batch sizes at 32K
    positions per request (identity block tables, every request of equal length, 32 q /
    8 KV heads). Each configuration rotates over enough layer pools that one graph replay
    streams at least 1 GiB, so the pools are not cache resident; per launch time from HIP
    events around the replays, and the fraction of 8 TB/s that the algorithmic bytes
    (visible positions x 4096 B + q and out) give."""
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.stack import capture_graph
    from synth import device as sdev, rng

    def one(view, B, n):
        mb = (n + 15) // 16
        keys = n if view == "full" else min(n, 2052)
        layers = max(2, -(-min_bytes // (B * keys * Hkv * 512)))
        bt = torch.arange(B * mb, dtype=torch.int32, device=device).view(B, mb)
        sl = torch.full((B,), n, dtype=torch.int32, device=device)
        caches = [ops.PagedKVCache(B * mb, B, Hq, Hkv, mb, block_tables=bt, seq_lens=sl, device=device)
                  for _ in range(layers)]
        for i, c in enumerate(caches):
            sdev.fill_normal_(c.k_pool, rng.mix_key(5, 1, i), 0)
            sdev.fill_normal_(c.v_pool, rng.mix_key(5, 2, i), 0)
        q = torch.randn(layers, B, Hq, 128, device=device)
        out = torch.zeros(layers, B, Hq, 128, device=device)
        ws = ops.workspace(B, Hq, device)
        if view == "full":
            fn = lambda: [ops.oda_decode_full(q[l], caches[l], out=out[l], ws=ws) for l in range(layers)]
        else:
            fn = lambda: [ops.oda_decode_local(q[l], caches[l], out=out[l], ws=ws) for l in range(layers)]
        g = capture_graph(fn)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * layers)
        nbytes = B * (keys * Hkv * 512 + 2 * Hq * 512)
        del g, caches
        torch.cuda.empty_cache()
        return {"view": view, "batch": B, "n": n, "us_per_launch": round(us, 2),
                "frac_of_peak": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 3)}

    def ragged_full(B, lo=4096, hi=131072):
        # a large batch of ragged lengths (log-uniform in [lo, hi], seeded), each request's
        # pages contiguous in one pool; one Full launch per replay (the pool exceeds 1 GiB)
        import math
        import numpy as np
        g = np.random.default_rng(np.random.SeedSequence([9, 7, B]))
        ns = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=B))).astype(np.int64)
        nbs = (ns + 15) // 16
        mb, total = int(nbs.max()), int(nbs.sum())
        bt = np.zeros((B, mb), np.int32)
        off = 0
        for b in range(B):
            bt[b, :nbs[b]] = np.arange(off, off + nbs[b])
            off += int(nbs[b])
        cache = ops.PagedKVCache(total, B, Hq, Hkv, mb, block_tables=torch.as_tensor(bt, device=device),
                                 seq_lens=torch.as_tensor(ns.astype(np.int32), device=device), device=device)
        sdev.fill_normal_(cache.k_pool, rng.mix_key(5, 1, 99), 0)
        sdev.fill_normal_(cache.v_pool, rng.mix_key(5, 2, 99), 0)
        q = torch.randn(B, Hq, 128, device=device)
        out = torch.zeros(B, Hq, 128, device=device)
        ws = ops.workspace(B, Hq, device)
        g2 = capture_graph(lambda: ops.oda_decode_full(q, cache, out=out, ws=ws))
        for _ in range(2):
            g2.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps // 2):
            g2.replay()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps // 2)
        nbytes = int(ns.sum()) * Hkv * 512 + B * 2 * Hq * 512
        del g2, cache
        torch.cuda.empty_cache()
        return {"view": "full", "batch": B, "n": "ragged %d-%d (log-uniform)" % (lo, hi), "us_per_launch": round(us, 2),
                "frac_of_peak": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 3)}

    cases = [("full", 1, n) for n in (4096, 16384, 32768, 65536, 131072, 262144)]
    cases += [("full", B, 32768) for B in (2, 4, 8, 12, 16, 24, 32)]
    cases += [("local", B, 32768) for B in (1, 8, 32, 64)]
    res = []
    for view, B, n in cases:
        res.append(one(view, B, n))
        log("sweep: %s" % json.dumps(res[-1]))
    for B in (96, 128):
        res.append(ragged_full(B))
        log("sweep: %s" % json.dumps(res[-1]))
    return res


def clock_ramp(device, ms):
    """Keeps the GPU busy with streaming reads (sk_stream_read over 1 GiB, launched in groups
    of 8) for about `ms` milliseconds of wall time, so that a short timed window does not
    start at the idle clocks the graph capture leaves behind. Touches no decode state."""
    import torch
    from sparse_kv_recall_amd import ops
    data = torch.ones(1 << 28, dtype=torch.int32, device=device)
    sink = ops.stream_read(data)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            ops.stream_read(data, sink)
        torch.cuda.synchronize()
    spent = (time.perf_counter() - t0) * 1e3
    del data, sink
    return spent


def stream_peak(device, gib=4, reps=5):
    """Measured streaming-read bandwidth: sk_stream_read over a 4 GiB buffer (16-byte
    non-temporal loads, 1 KiB contiguous per wave instruction, as the decode kernels
    issue them), median over `reps` groups of 4 launches queued back to back, timed with HIP
    events. The reference for the
    fraction of what this GPU streams in practice, beside the 8 TB/s of the data sheet."""
    import torch
    from sparse_kv_recall_amd import ops
    data = torch.ones(gib << 28, dtype=torch.int32, device=device)
    sink = ops.stream_read(data)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):  # launches queued back to back, so no host launch latency is timed
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(4):
            ops.stream_read(data, sink)
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1) / 4)
    ms = sorted(times)[len(times) // 2]
    nbytes = data.numel() * 4
    del data
    torch.cuda.empty_cache()
    return nbytes / (ms * 1e-3) / 1e9


def stream_floor(device, sizes, launches=36, reps=3):
    """Size-matched streaming reference: sk_stream_read launched `launches` times in one
    HIP graph, each launch over its own slice of the given size (as the decode launches
    rotate over 36 layers' pools, so no slice is still in the last-level cache). Per
    size, the time of one launch that does nothing but stream that many bytes, launch
    and ramp included: the floor for a decode launch that reads the same bytes."""
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.stack import capture_graph
    out = {}
    for name, nbytes in sizes:
        per = (int(nbytes) + 4095) // 4096 * 4096
        data = torch.ones(launches * per // 4, dtype=torch.int32, device=device)
        sink = torch.empty(ops.STREAM_READ_GRID, dtype=torch.int32, device=device)
        slices = [data[i * per // 4:(i + 1) * per // 4] for i in range(launches)]

        def run():
            for sl in slices:
                ops.stream_read(sl, sink)

        graph = capture_graph(run)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            graph.replay()
        e1.record()
        e1.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (reps * launches)
        gbs = per / (us * 1e-6) / 1e9
        out[name] = {"bytes": per, "us_per_launch": round(us, 2), "achieved_GBs": round(gbs, 1),
                     "frac": round(gbs / HBM_PEAK_GBS, 4)}
        del graph, slices, data
        torch.cuda.empty_cache()
    return out


def local_view_rate(stack, feeder, reps):
    """Per-launch time of the Local view over all layers at the current n: the step's Local
    pass (the tile-table launch and one Local launch per layer, each committing its
    candidate at n - 1) captured in one graph and timed with HIP events around the replays;
    the table launch's share is spread over the layers."""
    import torch
    from sparse_kv_recall_amd.stack import capture_graph
    q, k, v = feeder.q, feeder.k, feeder.v
    g = capture_graph(lambda: stack.local_pass(q[:, 0, :], k[:, 0, :], v[:, 0, :]))
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    e1.synchronize()
    del g
    return e0.elapsed_time(e1) / (reps * stack.layers)


def gated_off_launch(stack, feeder, reps=20):
    """Per-launch time of the recall pass's Full launches when the gate is 0, so that every
    workgroup leaves at once: the per-node cost that the step graph pays 36 times on
    every non-recall step (HIP graphs have no conditional node that could skip them)."""
    import torch
    from sparse_kv_recall_amd.stack import capture_graph
    q, k, v = feeder.q, feeder.k, feeder.v
    g = capture_graph(lambda: stack.full_pass(q[:, 1, :], k[:, 1, :], v[:, 1, :], gated=True))
    stack.gate.zero_()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1) / (reps * stack.layers)


def roofline_blocks(stack, feeder, reps, seed=11):
    """Block-list (Declarative-Attention) decode over the same 36 pools at the current n,
    through a seeded permutation of the block table, keeping (a) every block and (b) a
    seeded 12.5 % of the blocks plus the last one. Three graphs, each timed with HIP
    events per layer: da_decode_blocks in every layer (rewrite + attention), one
    da_gather per step and da_decode_gathered per layer, and the decode kernel alone;
    returns achieved GB/s of algorithmic bytes for each."""
    import numpy as np
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.stack import capture_graph
    c0 = stack.caches[0]
    n = int(stack.seq_lens[0].item())
    nb = (n + 15) // 16
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([3, 30, seed])))
    perm = np.full((1, c0.max_blocks), -1, np.int32)
    perm[0, :nb] = g.permutation(c0.num_phys_blocks)[:nb]
    bt = torch.as_tensor(perm, device="cuda")
    views = [ops.PagedKVCache(c.num_phys_blocks, 1, c.num_q_heads, c.num_kv_heads, c.max_blocks,
                              block_tables=bt, seq_lens=stack.seq_lens, k_pool=c.k_pool, v_pool=c.v_pool)
             for c in stack.caches]
    words = (c0.max_blocks + 31) // 32
    out = {}
    for name, frac in (("all_blocks", 1.0), ("keep_12.5pct", 0.125)):
        kept = np.arange(nb) if frac >= 1.0 else np.union1d(
            g.choice(nb, size=int(round(frac * nb)), replace=False), [nb - 1])
        mask = np.zeros(words, np.uint32)
        for b in kept:
            mask[b // 32] |= np.uint32(1 << (int(b) % 32))
        mt = torch.as_tensor(mask.view(np.int32)[None], device="cuda")
        gat = torch.zeros((1, c0.max_blocks), dtype=torch.int32, device="cuda")
        cnt = torch.zeros_like(gat)
        num = torch.zeros(1, dtype=torch.int32, device="cuda")
        positions = int(sum(min(16, n - 16 * int(b)) for b in kept))

        def per_call():  # the rewrite repeated in every layer's call
            for l, v in enumerate(views):
                ops.da_decode_blocks(feeder.q[l, 1], v, mt, scale=stack.scale, out=stack.out[l], gathered=gat,
                                     gathered_cnt=cnt, num_kept=num, ws=stack.ws)

        def per_step():  # one rewrite per step, one decode launch per layer
            ops.da_gather(views[0], mt, gathered=gat, gathered_cnt=cnt, num_kept=num, ws=stack.ws)
            for l, v in enumerate(views):
                ops.da_decode_gathered(feeder.q[l, 1], v, gat, cnt, num, scale=stack.scale, out=stack.out[l],
                                       ws=stack.ws)

        def decode_only():  # the block-list decode kernel alone, list already gathered
            for l, v in enumerate(views):
                ops.da_decode_gathered(feeder.q[l, 1], v, gat, cnt, num, scale=stack.scale, out=stack.out[l],
                                       ws=stack.ws)

        nbytes = positions * stack.Hkv * 128 * 4 + 2 * stack.Hq * 128 * 4
        res = {"kept_positions": positions}
        for key, fn in (("gather_in_every_call", per_call), ("gather_once_per_step", per_step),
                        ("decode_kernel", decode_only)):
            graph = capture_graph(fn)
            graph.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                graph.replay()
            e1.record()
            e1.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / (reps * len(views))
            res[key] = {"us_per_layer": round(us, 2), "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                        "frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            del graph
        out[name] = res
    return out


def kernel_source_hash():
    """Hash of the decode kernel's source with comments and whitespace removed, so that the
    counter summary stays valid across comment edits and is dropped on any code change."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in ("sparse_kv_recall_amd/csrc/decode.hip", "sparse_kv_recall_amd/csrc/sk_internal.h"):
        with open(os.path.join(ROOT, f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def profiled_traffic(bytes_now):
    """HBM bytes per Full-view launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE, each scaled by its copy-kernel calibration), rescaled
    from the profiled n to this launch's algorithmic bytes. None when the summary is
    missing or was taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", "decode_128k_hbm_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("#", "|", "`")):
                k, _, v = line.partition(":")
                vals[k.strip()] = v.strip()
    try:
        if vals["source_hash"] != kernel_source_hash():
            return None
        measured = (float(vals["full_fetch_kib"]) * float(vals["fetch_scale"]) +
                    float(vals["full_write_kib"]) * float(vals["write_scale"])) * 1024.0
        n_prof = int(vals["full_n"])
    except (KeyError, ValueError):
        return None
    alg_prof = n_prof * 8 * 128 * 4 + 2 * 32 * 128 * 4 + 2 * 8 * 128 * 2
    return measured * bytes_now / alg_prof


def copy_calibration(device):
    """A plain copy of known size (512 MiB) for scaling the HBM counters."""
    import torch
    a = torch.empty(256 << 20, dtype=torch.int16, device=device)
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    return a.numel() * 2


def cpu_baseline(wl, recall_rate, budget_s=20.0, local_s=2.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload at step 0
    (n = 131073), timed on the host cores: Local layer-steps (four layers' sinks and
    windows, each step with another step's candidates) for about `local_s` seconds, then
    Full layer-steps over one layer's whole history (each with another step's candidates)
    until about `budget_s` seconds of oracle time in all. Input generation is not timed.
    Tokens/s = 1 / (L * t_local + rate * L * t_full) with the mean times per layer-step."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = 1
    H0 = int(wl.H0[0])
    n = H0 + 1
    scale = 1.0 / math.sqrt(128.0)
    locals_ = []
    for l in range(4):  # the positions the Local view reads, per layer
        k = np.zeros((n, wl.Hkv, 128), np.uint16)
        v = np.zeros((n, wl.Hkv, 128), np.uint16)
        k[:4] = wl.hist_bits("k", l, 0, 4)
        v[:4] = wl.hist_bits("v", l, 0, 4)
        k[n - 2048:n - 1] = wl.hist_bits("k", l, n - 2048, 2047)
        v[n - 2048:n - 1] = wl.hist_bits("v", l, n - 2048, 2047)
        locals_.append((l, k, v))
    t_local, n_local = 0.0, 0
    while (t_local < local_s or n_local < 4) and n_local < 4096:
        l, k, v = locals_[n_local % 4]
        step = n_local // 4
        q = wl.cand_q(step, l, 0, 0)
        kn, vn = wl.cand_kv(step, l, 0, 0)
        t0 = time.perf_counter()
        oracle.oda.local_pass(q, kn, vn, k, v, n, scale)
        t_local += time.perf_counter() - t0
        n_local += 1
    del locals_
    layer_full = 1
    k = np.empty((n, wl.Hkv, 128), np.uint16)
    v = np.empty((n, wl.Hkv, 128), np.uint16)
    k[:H0] = wl.hist_bits("k", layer_full, 0, H0)
    v[:H0] = wl.hist_bits("v", layer_full, 0, H0)
    t_full, n_full = 0.0, 0
    while (t_local + t_full < budget_s or n_full < 1) and n_full < 256:
        q = wl.cand_q(n_full, layer_full, 1, 0)
        kn, vn = wl.cand_kv(n_full, layer_full, 1, 0)
        t0 = time.perf_counter()
        oracle.oda.full_pass(q, kn, vn, k, v, n, scale)
        t_full += time.perf_counter() - t0
        n_full += 1
    mean_local, mean_full = t_local / n_local, t_full / n_full
    step_s = wl.layers * mean_local + recall_rate * wl.layers * mean_full
    return {"value": 1.0 / step_s, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": ("fp64 oracle at n=131073: %d Local layer-steps (4 layers' sinks and windows, %.4f s each) "
                       "and %d Full layer-steps (layer %d's whole history, %.3f s each), each with another "
                       "step's candidates; %.1f s of oracle time; per-step time = 36*t_local + %.3f*36*t_full; "
                       "input generation not timed" % (n_local, mean_local, n_full, layer_full, mean_full,
                                                        t_local + t_full, recall_rate))}


def always_full_rate(stack, feeder, wl, steps):
    """Always-Full decoding on the same stack and kernels (every step attends all n keys
    and commits its candidate; no Local pass, no gate): the baseline ODA is set against.
    Replays the first `steps` steps again."""
    import torch
    from sparse_kv_recall_amd.stack import capture_graph
    q, k, v = feeder.q, feeder.k, feeder.v

    def step():
        feeder.step()
        stack.full_pass(q[:, 1, :], k[:, 1, :], v[:, 1, :], gated=False)

    graph = capture_graph(step)
    feeder.set_step(0)
    graph.replay()
    torch.cuda.synchronize()
    feeder.set_step(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    del graph
    return {"steps": steps, "tok_s": round(steps * wl.batch / (ms / 1e3), 2), "ms_per_step": round(ms / steps, 4)}


def _stage_history(cache, wl, unit, H0, request, device):
    """Seeded bf16 history of one request (positions 0 .. H0-1), written into its pages."""
    import torch
    from sparse_kv_recall_amd import ops
    from synth import device as sdev
    from synth.workloads import C_KHIST, C_VHIST
    stage_k = torch.empty((H0, wl.Hkv, 128), dtype=torch.bfloat16, device=device)
    stage_v = torch.empty_like(stage_k)
    sdev.fill_normal_(stage_k, wl.key(C_KHIST, unit), 0)
    sdev.fill_normal_(stage_v, wl.key(C_VHIST, unit), 0)
    ops.kv_write(cache, request, 0, stage_k, stage_v)


def _time_replays(graph, steps, reset, reps):
    """Best of `reps` passes of `steps` graph replays (reset() before each), in ms."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = None
    for _ in range(reps):
        reset()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return best


def other_workloads(device, reps=2):
    """Throughput of the other seeded workloads, each step one HIP graph replay, all
    steps from step 0 (best of `reps` passes; inputs resident before timing):
    * oda_stack16k: 28 layers, 16 q / 8 KV heads, 16K history, the fp32 recall head
      deciding on the device -- tokens/s, the recall steps it chose, and the Full view
      over all 28 layers at the final n (1.9 GB per rotation, more than the MALL holds);
    * da_32k: declared mode -> keep mask -> gathered list -> attention over the kept
      blocks, 32K context, permuted pool -- microseconds per step for each mode (events
      around every replay of one pass), and the same with the block-table rewrite done
      inside the decode kernel (da_decode_declared);
    * ragged32: 32 requests of 4K-128K, each step Full or the request's fallback (Local
      or its keep-list) -- tokens/s and GB/s of the attended positions (4096 B each), with
      the three views in one decode launch, and tokens/s with one launch per view."""
    import numpy as np
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.stack import DAStep, ODAStack, RaggedBatch, capture_graph
    from synth import device as sdev
    from synth import workloads

    res = {}
    # ---- 16K stack with the recall head
    wl = workloads.oda_stack16k()
    H0 = int(wl.H0[0])
    seq = torch.zeros(1, dtype=torch.int32, device=device)
    stack = ODAStack(wl.layers, 1, wl.Hq, wl.Hkv, wl.num_phys_blocks, wl.max_blocks,
                     torch.as_tensor(wl.block_tables, device=device), seq, sinks=wl.sinks, window=wl.window,
                     device=device)
    for l in range(wl.layers):
        _stage_history(stack.caches[l], wl, l, H0, 0, device)
    feeder = sdev.Feeder(wl, seq, device=device, with_x=True)
    W = tuple(torch.as_tensor(a, device=device) for a in wl.recall_weights())

    def step16k():
        feeder.step()
        stack.local_pass(feeder.q[:, 0], feeder.k[:, 0], feeder.v[:, 0])
        stack.gate_from_recall_head(feeder.x, *W, theta=wl.theta)
        stack.full_pass(feeder.q[:, 1], feeder.k[:, 1], feeder.v[:, 1], gated=True)

    graph = capture_graph(step16k)
    feeder.set_step(0)
    recalls = 0
    for _ in range(wl.steps):  # untimed pass: the head's decisions
        graph.replay()
        recalls += int(stack.gate[0].item())
    ms = _time_replays(graph, wl.steps, lambda: feeder.set_step(0), reps)
    n_end = int(seq[0].item())
    # the Full view of every layer at the last step's n, ungated, as a graph (eager launches
    # from Python would be timed at the host's launch rate, not the kernel's)
    full_graph = capture_graph(lambda: stack.full_pass(feeder.q[:, 1], feeder.k[:, 1], feeder.v[:, 1], gated=False))
    full_graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        full_graph.replay()
    e1.record()
    e1.synchronize()
    full_us = e0.elapsed_time(e1) * 1e3 / (3 * wl.layers)
    del full_graph
    full_bytes = n_end * wl.Hkv * 512 + 2 * wl.Hq * 512 + wl.Hkv * 512
    res["oda_stack16k"] = {"steps": wl.steps, "recall_steps": recalls, "tok_s": round(wl.steps / (ms / 1e3), 1),
                           "ms_per_step": round(ms / wl.steps, 4), "full_view_us": round(full_us, 2),
                           "full_view_frac_of_peak": round(full_bytes / (full_us * 1e-6) / (HBM_PEAK_GBS * 1e9), 3),
                           "full_view_n": n_end}
    del graph, stack, feeder
    torch.cuda.empty_cache()

    # ---- 32K DA workload, per declared mode
    wl = workloads.da_32k()
    H0 = int(wl.H0[0])
    seq = torch.zeros(1, dtype=torch.int32, device=device)
    cache = ops.PagedKVCache(wl.num_phys_blocks, 1, wl.Hq, wl.Hkv, wl.max_blocks,
                             block_tables=torch.as_tensor(wl.block_tables, device=device), seq_lens=seq,
                             device=device)
    _stage_history(cache, wl, 0, H0, 0, device)
    feeder = sdev.Feeder(wl, seq, device=device, with_decl=True)
    modes = wl.decl[:, 0, 0]
    res["da_32k"] = {"steps": wl.steps}
    for suffix, in_kernel in (("", False), ("_rewrite_in_kernel", True)):
        da = DAStep(cache, wl.da_local_tokens, device=device, in_kernel_rewrite=in_kernel)

        def step_da():
            feeder.step()
            da.step(feeder.q[0, 0], feeder.k[0, 0], feeder.v[0, 0], feeder.decl)

        graph = capture_graph(step_da)
        ms = _time_replays(graph, wl.steps, lambda: feeder.set_step(0), reps)
        feeder.set_step(0)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(wl.steps)]
        for a, b in ev:
            a.record()
            graph.replay()
            b.record()
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])
        res["da_32k"]["us_per_step" + suffix] = round(ms * 1e3 / wl.steps, 2)
        res["da_32k"]["us_per_step_by_mode" + suffix] = {
            name: round(float(np.median(per[modes == m])), 2) for m, name in ((0, "global"), (1, "focus"), (2, "local"))}
        del graph, da
    del cache, feeder
    torch.cuda.empty_cache()

    # ---- ragged batch of 32
    wl = workloads.ragged32()
    seq = torch.zeros(wl.batch, dtype=torch.int32, device=device)
    cache = ops.PagedKVCache(wl.num_phys_blocks, wl.batch, wl.Hq, wl.Hkv, wl.max_blocks,
                             block_tables=torch.as_tensor(wl.block_tables, device=device), seq_lens=seq,
                             device=device)
    for r in range(wl.batch):
        _stage_history(cache, wl, r, int(wl.H0[r]), r, device)
    rb = RaggedBatch(cache, torch.as_tensor(wl.fallback, device=device),
                     torch.as_tensor(wl.keep_mask.view(np.int32), device=device), sinks=wl.sinks,
                     window=wl.window, device=device)
    feeder = sdev.Feeder(wl, seq, device=device, with_scores=True)

    def step_ragged():
        feeder.step()
        rb.step(feeder.q[0, 0], feeder.k[0, 0], feeder.v[0, 0], feeder.scores, wl.theta)

    # the three views in one decode launch (the default), then one selector launch per view
    graph = capture_graph(step_ragged)
    ms = _time_replays(graph, wl.steps, lambda: feeder.set_step(0), reps)
    del graph
    rb.one_launch = False
    graph = capture_graph(step_ragged)
    ms_three = _time_replays(graph, wl.steps, lambda: feeder.set_step(0), reps)
    # attended positions per step and request: n (Full), min(n, sinks + window) (Local), or
    # the positions of the kept blocks below n (keep-list)
    scores = wl.scores_all()
    bits = np.unpackbits(wl.keep_mask.view(np.uint8), axis=1, bitorder="little")
    positions, recalls = 0, 0
    for t in range(wl.steps):
        for r in range(wl.batch):
            n = int(wl.H0[r]) + t + 1
            if scores[t, r] > wl.theta:
                positions += n
                recalls += 1
            elif wl.fallback[r] == ops.MODE_LOCAL:
                positions += min(n, wl.sinks + wl.window)
            else:
                nb = (n + 15) // 16
                kept = np.nonzero(bits[r, :nb])[0]
                positions += int(np.minimum(16, n - 16 * kept).sum())
    nbytes = positions * wl.Hkv * 512
    res["ragged32"] = {"steps": wl.steps, "batch": wl.batch, "full_request_steps": recalls,
                       "tok_s": round(wl.steps * wl.batch / (ms / 1e3), 1), "ms_per_step": round(ms / wl.steps, 4),
                       "attention_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "frac_of_peak": round(nbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 3),
                       "views": "one launch for the three views (oda_decode_views)",
                       "tok_s_one_launch_per_view": round(wl.steps * wl.batch / (ms_three / 1e3), 1)}
    del graph, cache, rb, feeder
    torch.cuda.empty_cache()
    return res


def config_lines(device, reps=3, min_bytes=1 << 30):
    """Per-configuration figures beside the metric:
    * oda_small (1 layer, 8 q / 2 KV heads, 4K history, 64 steps, Full on a seeded
      Bernoulli(0.4) step): microseconds per step, each step one graph replay (feed,
      Local, gate, gated Full). 4 MiB of KV stay cache resident: a latency figure.
    * da_32k's three declared modes at the first step (n = 32769, the block list gathered
      through the device's keep mask), each attended over enough pools that the attended
      bytes of one graph replay reach `min_bytes` (at least 8 pools), so the last-level
      cache cannot serve them: microseconds per launch and GB/s of attended positions
      (4096 B each, plus q and out), with the commit of the current token."""
    import math as _m

    import numpy as np
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.stack import ODAStack, capture_graph
    from synth import device as sdev
    from synth import rng
    from synth import workloads

    res = {}
    wl = workloads.oda_small()
    H0 = int(wl.H0[0])
    seq = torch.zeros(1, dtype=torch.int32, device=device)
    stack = ODAStack(wl.layers, 1, wl.Hq, wl.Hkv, wl.num_phys_blocks, wl.max_blocks,
                     torch.as_tensor(wl.block_tables, device=device), seq, sinks=wl.sinks, window=wl.window,
                     device=device)
    _stage_history(stack.caches[0], wl, 0, H0, 0, device)
    feeder = sdev.Feeder(wl, seq, device=device, with_scores=True)

    def step_small():
        feeder.step()
        stack.local_pass(feeder.q[:, 0], feeder.k[:, 0], feeder.v[:, 0])
        stack.gate_from_scores(feeder.scores, wl.theta)
        stack.full_pass(feeder.q[:, 1], feeder.k[:, 1], feeder.v[:, 1], gated=True)

    graph = capture_graph(step_small)
    ms = _time_replays(graph, wl.steps, lambda: feeder.set_step(0), reps)
    res["oda_small"] = {"steps": wl.steps, "recall_steps": int((wl.sched_scores[:, 0] > 0).sum()),
                        "us_per_step": round(ms * 1e3 / wl.steps, 2),
                        "note": "4 MiB of KV, cache resident: latency, no HBM claim"}
    del graph, stack, feeder
    torch.cuda.empty_cache()

    wl = workloads.da_32k()
    n = int(wl.H0[0]) + 1
    mb = wl.max_blocks
    seq = torch.full((1,), n, dtype=torch.int32, device=device)
    ident = torch.arange(mb, dtype=torch.int32, device=device)[None]
    probe = ops.PagedKVCache(1, 1, wl.Hq, wl.Hkv, mb, block_tables=ident, seq_lens=seq, device=device)
    ws = ops.workspace(1, wl.Hq, device)
    modes = {}
    for mode, name in ((ops.DA_GLOBAL, "global"), (ops.DA_FOCUS, "focus"), (ops.DA_LOCAL, "local")):
        first = int(np.flatnonzero(wl.decl[:, 0, 0] == mode)[0])
        decl = torch.as_tensor(wl.decl[first], device=device)
        mask = ops.da_keep_mask(decl, probe, wl.da_local_tokens)
        gat, cnt, num = ops.da_gather(probe, mask, ws=ws)  # identity table: the kept logical blocks
        K = int(num[0].item())
        kept = gat[0, :K].cpu().numpy()
        positions = int(cnt[0, :K].sum().item())
        nbytes = positions * wl.Hkv * 512 + 2 * wl.Hq * 512
        P = max(8, -(-min_bytes // nbytes))
        kpool = torch.empty((P * K, wl.Hkv, 2048), dtype=torch.bfloat16, device=device)
        vpool = torch.empty_like(kpool)
        sdev.fill_normal_(kpool, rng.mix_key(4, 40, mode), 0)
        sdev.fill_normal_(vpool, rng.mix_key(4, 41, mode), 0)
        views, lists = [], []
        for p in range(P):
            bt = np.zeros((1, mb), np.int32)
            bt[0, kept] = p * K + np.arange(K, dtype=np.int32)
            c = ops.PagedKVCache(P * K, 1, wl.Hq, wl.Hkv, mb, block_tables=torch.as_tensor(bt, device=device),
                                 seq_lens=seq, k_pool=kpool, v_pool=vpool)
            views.append(c)
            lists.append(ops.da_gather(c, mask, ws=ws))
        q = torch.randn(P, 1, wl.Hq, 128, device=device)
        kn = torch.randn(P, 1, wl.Hkv, 128, device=device).to(torch.bfloat16)
        vn = torch.randn(P, 1, wl.Hkv, 128, device=device).to(torch.bfloat16)
        out = torch.zeros(P, 1, wl.Hq, 128, device=device)

        def run():
            for p in range(P):
                g_, c_, n_ = lists[p]
                ops.da_decode_gathered(q[p], views[p], g_, c_, n_, kn[p], vn[p], out=out[p], ws=ws)

        graph = capture_graph(run)
        ms = _time_replays(graph, 4, lambda: None, reps)
        us = ms * 1e3 / (4 * P)
        modes[name] = {"kept_blocks": K, "kept_positions": positions, "pools": P,
                       "attended_bytes_per_replay": P * nbytes, "us_per_launch": round(us, 2),
                       "achieved_GBs": round(nbytes / (us * 1e-6) / 1e9, 1),
                       "frac": round(nbytes / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4)}
        log("da_32k %s over %d pools: %s" % (name, P, json.dumps(modes[name])))
        del graph, views, lists, kpool, vpool
        torch.cuda.empty_cache()
    res["da_32k_modes_rotated"] = dict(modes, note="n = 32769 (step 0), permuted-table lists from the device's "
                                                   "keep mask; pools rotated so one replay attends >= 1 GiB")
    return res


def da_tags_rate(device, reps=2):
    """Declaration-driven DA decode at 32K (the ``da_tags_32k`` workload): per step the
    input token advances the device parser (declaration + keep mask), then the kept
    blocks are gathered and attended; and the same with the parser writing only the
    declaration and the decode kernel deriving the kept blocks from it. Returns the
    average step time over the 512 steps of each."""
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.stack import DATagStep, capture_graph
    from synth import device as sdev
    from synth import workloads
    from synth.workloads import C_KHIST, C_VHIST

    wl = workloads.da_tags_32k()
    H0 = int(wl.H0[0])
    seq = torch.zeros(1, dtype=torch.int32, device=device)
    cache = ops.PagedKVCache(wl.num_phys_blocks, 1, wl.Hq, wl.Hkv, wl.max_blocks,
                             block_tables=torch.as_tensor(wl.block_tables, device=device), seq_lens=seq)
    stage_k = torch.empty((H0, wl.Hkv, 128), dtype=torch.bfloat16, device=device)
    stage_v = torch.empty_like(stage_k)
    sdev.fill_normal_(stage_k, wl.key(C_KHIST, 0), 0)
    sdev.fill_normal_(stage_v, wl.key(C_VHIST, 0), 0)
    ops.kv_write(cache, 0, 0, stage_k, stage_v)
    feeder = sdev.Feeder(wl, seq, device=device, with_tokens=True)
    res = {"workload": "da_tags_32k: 1 layer, 32 q / 8 kv heads, context 32768 + 512 steps, declarations "
                       "parsed on the device from a seeded token stream", "steps": wl.steps}
    for key, in_kernel in (("us_per_step", False), ("us_per_step_rewrite_in_kernel", True)):
        da = DATagStep(cache, wl.da_tags, torch.as_tensor(wl.output_begin, device=device),
                       segments=torch.as_tensor(wl.segments, device=device), local_tokens=wl.da_local_tokens,
                       in_kernel_rewrite=in_kernel)

        def step():
            feeder.step()
            da.step(feeder.q[0, 0], feeder.k[0, 0], feeder.v[0, 0], feeder.tokens)

        graph = capture_graph(step)
        graph.replay()
        torch.cuda.synchronize()

        def reset():
            feeder.set_step(0)
            da.state.zero_()

        res[key] = round(_time_replays(graph, wl.steps, reset, reps) * 1e3 / wl.steps, 2)
        del graph
    return res


def decoder_rates(device, contexts=(4096, 131072), steps=64, recalls=8):
    """Whole-model decode (Qwen3-1.7B's dense shape, random weights): the ODA step
    (Local pass through all 28 layers, recall head on its final hidden state, gated
    recall pass, select) against always-Full decoding on the same kernels, at two
    history lengths. The recall decisions follow a seeded schedule of `recalls` in
    `steps` (the head's score is still computed every step), so both contexts see the
    pages' 12.5 % rate. KV pools are filled with random bf16 (a random history)."""
    import numpy as np
    import torch
    from sparse_kv_recall_amd import ops
    from sparse_kv_recall_amd.model import DecoderShape, ODADecoder
    from sparse_kv_recall_amd.stack import HostRoutedStep, capture_graph
    from synth import device as sdev
    from synth.decoder import decoder_qwen3_1_7b
    from synth.workloads import np_rng

    out = {}
    for H0 in contexts:
        wl = decoder_qwen3_1_7b(H0, steps)
        mb = wl.max_blocks
        seq = torch.full((1,), H0, dtype=torch.int32, device=device)
        bt = torch.arange(mb, dtype=torch.int32, device=device)[None]
        caches = [ops.PagedKVCache(mb, 1, wl.q_heads, wl.kv_heads, mb, block_tables=bt, seq_lens=seq, device=device)
                  for _ in range(wl.layers)]
        for l, c in enumerate(caches):
            sdev.fill_normal_(c.k_pool, wl.hist_key("k", l), 0)
            sdev.fill_normal_(c.v_pool, wl.hist_key("v", l), 0)
        shape = DecoderShape(wl.layers, wl.hidden, wl.q_heads, wl.kv_heads, wl.intermediate, wl.vocab,
                             wl.recall_hidden)
        model = ODADecoder(shape, wl.device_weights(device), caches, device=device)
        tokens = torch.as_tensor(wl.tokens.astype(np.int64), device=device)
        sched = -np.ones(steps, np.float32)
        sched[np_rng(wl.wid, 99).choice(steps, size=recalls, replace=False)] = 1.0
        sched = torch.as_tensor(sched, device=device)
        t_idx = torch.zeros(1, dtype=torch.int64, device=device)
        score = torch.zeros(1, dtype=torch.float32, device=device)

        def feed():
            model.token.copy_(torch.index_select(tokens, 0, t_idx))
            score.copy_(torch.index_select(sched, 0, t_idx))
            seq.add_(1)
            t_idx.add_(1)

        def oda_step():
            feed()
            model.local_pass()
            model.recall_gate(0.0)
            ops.oda_gate_scores(score, 0.0, out=model.gate)  # the schedule decides
            model.recall_pass(gated=True)
            ops.select(model.gate, model.final_full, model.h_local_final, model.h_prev)

        def full_step():
            feed()
            model.always_full_step()

        def oda_first():
            feed()
            model.local_pass()
            model.recall_gate(0.0)
            ops.oda_gate_scores(score, 0.0, out=model.gate)

        def oda_recall():
            model.recall_pass(gated=True)
            oda_select()

        def oda_select():
            ops.select(model.gate, model.final_full, model.h_local_final, model.h_prev)

        res = {}
        for name, fn in (("oda", oda_step), ("always_full", full_step), ("oda_host_routed", None)):
            if fn is None:
                graph = HostRoutedStep(oda_first, oda_recall, model.gate, skip=oda_select)
            else:
                graph = capture_graph(fn)
            seq.fill_(H0)
            t_idx.zero_()
            for _ in range(4):  # warm replays, then back to step 0
                graph.replay()
            seq.fill_(H0)
            t_idx.zero_()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / steps
            del graph
        out["ctx_%d" % H0] = {"oda_ms_per_step": round(res["oda"], 4), "oda_tok_s": round(1e3 / res["oda"], 2),
                              "always_full_ms_per_step": round(res["always_full"], 4),
                              "always_full_tok_s": round(1e3 / res["always_full"], 2),
                              "oda_speedup": round(res["always_full"] / res["oda"], 3),
                              "host_routed_oda_ms_per_step": round(res["oda_host_routed"], 4),
                              "host_routed_oda_tok_s": round(1e3 / res["oda_host_routed"], 2),
                              "host_routed_oda_speedup": round(res["always_full"] / res["oda_host_routed"], 3),
                              "recall_steps": recalls, "steps": steps}
        del model, caches
        torch.cuda.empty_cache()
    return dict(out, model="Qwen3-1.7B dense shape (28 layers, hidden 2048, 16/8 heads, MLP 6144), random bf16 "
                           "weights, batch 1")


def hybrid_rate(stack, feeder, wl, steps):
    """Decode rate of the same workload with per-layer access control: three of every
    four layers restricted to the Local range (their recall pass runs the Local view).
    Replays the first `steps` steps again (rewriting the positions they committed)."""
    import torch

    saved = stack.local_only
    stack.local_only = frozenset(l for l in range(wl.layers) if l % 4 != 3)
    graph = capture_step(stack, feeder)
    feeder.set_step(0)
    graph.replay()
    torch.cuda.synchronize()
    feeder.set_step(0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    stack.local_only = saved
    del graph
    return {"local_only_layers": sum(1 for l in range(wl.layers) if l % 4 != 3),
            "steps": steps, "recall_steps": int((wl.sched_scores[:steps, 0] > 0).sum()),
            "tok_s": round(steps * wl.batch / (ms / 1e3), 2), "ms_per_step": round(ms / steps, 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--roofline-reps", type=int, default=3)
    ap.add_argument("--ramp-ms", type=float, default=300.0,
                    help="milliseconds of streaming reads before the warmup steps (GPU clock ramp; 0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-model", action="store_true", help="skip the weight-bearing decode measurement")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the throughput of the 16K stack, the 32K DA workload and the ragged batch")
    ap.add_argument("--sweep", action="store_true",
                    help="also sweep the Full and Local views over context lengths and batch sizes")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the decode path here is built and measured on a single "
              "MI355X (requests would shard across GPUs with no exchange, one long sequence by KV head); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from synth import workloads
    from synth.device import Feeder

    device = "cuda"
    torch.cuda.init()
    wl = workloads.oda_stack128k()
    if args.steps < RECALL_PERIOD or args.steps > wl.steps:
        print("--steps must be in %d..%d: the timed window starts at step 0 and needs a whole run of %d steps "
              "(one recall step and seven others)" % (RECALL_PERIOD, wl.steps, RECALL_PERIOD), file=sys.stderr)
        sys.exit(2)
    if args.ramp_ms > 0:  # the reference below is short too: measured at working clocks
        clock_ramp(device, args.ramp_ms)
    stream_gbs = stream_peak(device)  # before the stack is staged: a fresh allocation
    log("streaming-read reference: %.0f GB/s" % stream_gbs)
    log("staging %d layers x %d positions of bf16 KV" % (wl.layers, int(wl.H0[0])))
    t0 = time.time()
    stack = build_stack(wl, device)
    feeder = Feeder(wl, stack.seq_lens, device=device, with_scores=True)
    log("staged in %.1f s; capturing the step graph" % (time.time() - t0))
    graph = capture_step(stack, feeder)

    # A window of 20 steps lasts ~16 ms: started straight after the graph capture (GPU idle),
    # it ran 2-3 % below the steady rate of all 1024 steps (recall steps 3.48 against 3.34 ms
    # in one comparison); untimed streaming reads first bring it to that rate.
    ramp_ms = clock_ramp(device, args.ramp_ms) if args.ramp_ms > 0 else 0.0
    if ramp_ms:
        log("clock ramp: %.0f ms of streaming reads before the warmup steps" % ramp_ms)
    for _ in range(args.warmup):
        graph.replay()
    feeder.set_step(0)
    torch.cuda.synchronize()
    log("warmup done; timing %d steps" % args.steps)

    # one event between consecutive replays: the time of every step of the window
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record()
    for i in range(args.steps):
        graph.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per_step = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    ms_total = ev[0].elapsed_time(ev[-1])
    rec = wl.sched_scores[:args.steps, 0] > 0
    recalls = int(rec.sum())
    # The metric's rate is one recall step in eight. The window from step 0 holds exactly
    # that when --steps is a multiple of 8; otherwise it holds a few recalls more or less,
    # so the step time is the window's mean recall-step and non-recall-step times
    # weighted 1 : 7 (equal to the plain mean for whole runs of 8).
    ms_rec, ms_non = float(per_step[rec].mean()), float(per_step[~rec].mean())
    ms_per_step = (ms_rec + (RECALL_PERIOD - 1) * ms_non) / RECALL_PERIOD
    tok_s = wl.batch / (ms_per_step / 1e3)
    tok_s_window = args.steps * wl.batch / (ms_total / 1e3)
    assert torch.isfinite(stack.out).all().item(), "non-finite decode output"
    log("timed: %.3f ms/step at 1 recall in 8 (%.1f tok/s; recall steps %.3f ms, others %.3f ms); window of %d "
        "steps with %d recalls: %.1f tok/s, wall %.2f s" % (ms_per_step, tok_s, ms_rec, ms_non, args.steps, recalls,
                                                          tok_s_window, wall))

    # dominant kernel: the Full view at the last step's n, every layer, no gate
    n_now = int(stack.seq_lens[0].item())
    full_ms = roofline_full(stack, feeder, args.roofline_reps)
    bytes_full = n_now * wl.Hkv * 128 * 2 * 2 + 2 * wl.Hq * 128 * 4 + 2 * wl.Hkv * 128 * 2
    achieved = bytes_full / (full_ms * 1e-3) / 1e9
    log("Full-view kernel at n=%d: %.1f us per launch, %.0f GB/s" % (n_now, full_ms * 1e3, achieved))
    local_ms = local_view_rate(stack, feeder, 10)
    local_pos = min(n_now, wl.sinks + wl.window)
    bytes_local = local_pos * wl.Hkv * 128 * 2 * 2 + 2 * wl.Hq * 128 * 4 + 2 * wl.Hkv * 128 * 2
    log("Local-view kernel (%d positions, tile table): %.2f us per launch, %.0f GB/s"
        % (local_pos, local_ms * 1e3, bytes_local / (local_ms * 1e-3) / 1e9))
    gated_off_ms = gated_off_launch(stack, feeder)
    log("gated-off Full launch: %.2f us" % (gated_off_ms * 1e3))
    blocks = roofline_blocks(stack, feeder, args.roofline_reps)
    log("block-list view: %s" % json.dumps(blocks))
    floor = stream_floor(device, [("local_2052_positions", min(n_now, wl.sinks + wl.window) * wl.Hkv * 512),
                                  ("keep_12.5pct_positions", blocks["keep_12.5pct"]["kept_positions"] * wl.Hkv * 512),
                                  ("full_n", n_now * wl.Hkv * 512)])
    log("size-matched streaming reference: %s" % json.dumps(floor))
    host_routed = host_routed_rate(stack, feeder, wl, args.steps, min(args.warmup, 8))
    log("host-routed recall branch: %s" % json.dumps(host_routed))
    full_only = always_full_rate(stack, feeder, wl, min(64, args.steps))
    log("always-Full baseline: %s" % json.dumps(full_only))
    hybrid = hybrid_rate(stack, feeder, wl, min(256, args.steps))
    log("hybrid access control: %s" % json.dumps(hybrid))
    da_tags = da_tags_rate(device)
    log("declaration-driven DA step: %s" % json.dumps(da_tags))
    if not args.no_model:
        whole_model = decoder_rates(device)
        log("weight-bearing decode: %s" % json.dumps(whole_model))
    else:
        whole_model = None
    traffic = profiled_traffic(bytes_full)
    traffic = None if traffic is None else int(round(traffic))
    copy_calibration(device)

    # step bytes (algorithmic): Local reads min(n, 2052) positions per layer, Full n on
    # recall steps; per step at the 1 : 7 weighting of the value above
    ns = wl.H0[0] + 1 + np.arange(args.steps)
    bpt = wl.Hkv * 128 * 4
    local_b = float((wl.layers * np.minimum(ns, wl.sinks + wl.window) * bpt).mean())
    full_b = float((wl.layers * ns * bpt).mean())
    step_bytes = local_b + full_b / RECALL_PERIOD
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    full_bytes = full_b  # always-Full reads every key of every layer each step

    res = {
        "metric": METRIC,
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 KV; q and softmax weights enter the matrix cores as bf16 high+low pairs (~16 "
                 "significant bits), fp32 accumulate and softmax",
        "data": "synthetic (seeded counter-based N(0,1)-like values; no dataset or trained weights)",
        "config": {"workload": "oda_stack128k: 36 layers, 32 q / 8 kv heads, head_dim 128, history 131072 "
                               "+1 per step, batch 1, local s=4 w=2048, recall rate 12.5 %% (one seeded step in "
                               "every aligned run of 8); value = 1 / (mean recall-step time + 7 x mean other-step "
                               "time) x 8 over the timed window of %d steps from step 0, which holds %d recall "
                               "steps (%.4f)" % (args.steps, recalls, recalls / args.steps),
                   "recall_rate": 1.0 / RECALL_PERIOD,
                   "window": {"steps": args.steps, "recall_steps": recalls,
                              "recall_fraction": round(recalls / args.steps, 4),
                              "tok_s": round(tok_s_window, 2), "ms_per_step": round(ms_total / args.steps, 4),
                              "recall_step_ms": round(ms_rec, 4), "other_step_ms": round(ms_non, 4)},
                   "global_batch": 1, "seq_len": int(ns[-1]), "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "stream_peak_gbs": round(stream_gbs, 1),
                     "frac_of_stream_peak": round(achieved / stream_gbs, 4),
                     "kernel": "decode_kernel<full> (oda_decode_full), n=%d, 36-layer rotation" % n_now,
                     "us_per_launch": round(full_ms * 1e3, 2), "algorithmic_bytes_per_launch": int(bytes_full),
                     "traffic_source": "profiles/decode_128k_hbm_counters.md (rocprofv3 FETCH_SIZE x2.0 + "
                                       "WRITE_SIZE x1.0, rescaled to this n); null if the kernel changed"},
        "local_view": {"us_per_launch": round(local_ms * 1e3, 2), "positions": local_pos,
                       "algorithmic_bytes_per_launch": int(bytes_local),
                       "achieved_GBs": round(bytes_local / (local_ms * 1e-3) / 1e9, 1),
                       "frac": round(bytes_local / (local_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "stream_floor_us": floor["local_2052_positions"]["us_per_launch"],
                       "kernel": "decode_kernel<local, tile table> (oda_decode_local_tiles) in the step's Local "
                                 "pass graph (one table launch and 36 Local launches), n=%d" % n_now},
        "roofline_block_sparse": dict(blocks, kernel="decode_kernel<list> over a permuted block table (36-layer "
                                      "rotation, n=%d); also per layer with the rewrite (gather) in every call and "
                                      "once per step" % n_now),
        "clock_ramp_ms": round(ramp_ms, 1),
        "stream_floor": dict(floor, note="sk_stream_read alone, 36 launches over distinct slices in one graph, "
                                         "at the K/V bytes of the Local view, the 12.5 % block list and the Full "
                                         "view: what a launch that only streams those bytes costs"),
        "always_full_baseline": dict(full_only, speedup_of_oda=round(tok_s / full_only["tok_s"], 3),
                                     attention_bytes_ratio=round(float(full_bytes / step_bytes), 3)),
        "dispatch": {"graph_launches_per_step": 3 + 2 * wl.layers,
                     "gated_off_full_launch_us": round(gated_off_ms * 1e3, 2),
                     "gated_off_us_per_nonrecall_step": round(gated_off_ms * 1e3 * wl.layers, 1),
                     "note": "one feed, the Local tile table, 36 Local, the gate and 36 gated Full launches per step; on a "
                             "non-recall step the Full launches exit at once but each still costs a graph node"},
        "host_routed": dict(host_routed, note="the same step as two graphs split at the gate: the host reads the "
                                              "gate back and replays the 36 Full launches only on recall steps "
                                              "(no graph nodes for skipped launches; one host round trip per "
                                              "step)"),
        "hybrid_local_only": hybrid,
        "da_declared_step": da_tags,
        "whole_model_decode": whole_model,
        "step_hbm_gbs": round(float(step_gbs), 1),
        "wall_s_timed": round(wall, 3),
    }
    del graph, feeder, stack
    torch.cuda.empty_cache()
    if not args.no_other:
        res["other_workloads"] = other_workloads(device)
        log("other workloads: %s" % json.dumps(res["other_workloads"]))
        res["config_lines"] = config_lines(device)
        log("config lines: %s" % json.dumps(res["config_lines"]))
    if args.sweep:  # after the metric stack is freed: fresh pools, as in a process of their own
        res["view_sweep"] = view_sweep(device)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host (bounded sample)")
        res["cpu_baseline"] = cpu_baseline(wl, 1.0 / RECALL_PERIOD)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
