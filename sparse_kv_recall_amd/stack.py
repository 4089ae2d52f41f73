"""Decode-step drivers: the order in which one step calls the C ABI.

ODA step (On-Demand Attention summary page, "Approach"; Figure 1 caption):
  1. every layer runs the Local view, committing its candidate KV at n-1;
  2. the recall score gives the gate on the device (recall-head GEMV, or given scores);
  3. every layer runs the Full view gated by that flag: its workgroups exit at once
     when the gate is 0, otherwise it commits the Full candidate (overwriting the
     Local one) and overwrites the layer's output with the Full result.
The step never reads the gate on the host, so it can be captured once as a HIP
graph and replayed ("Developer perspective": one GPU execution flow).

Host-routed form (HostRoutedStep): the same launches in two graphs, split at the gate.
The host reads the gate back (4 bytes per request) and replays the recall-pass graph only
when some request is selected. Its launches still carry the device gate as their
selector, so the results are those of the one-graph step. Without a conditional graph
node, every skipped launch of the one-graph step still costs a graph node, and the
readback costs one host round trip per step instead.

Per-layer access control ("Developer perspective", the note on hybrid backbones: the
runtime may restrict chosen layers to the Local range): a layer marked local-only runs
its Local view in step 3 as well, under the same gate, so it never reads beyond the
sinks and the window; the recall pass's candidate is still the one committed.

Ragged-batch step: a per-request view is chosen on the device from the scores
(Full when score > theta, else the request's fallback), then the three views are
launched with selectors, each request being served by exactly one of them.

This module only sequences library calls; it computes nothing itself.
"""

import math

import numpy as np
import torch

from . import ops


class ODAStack:
    """Paged caches of an L-layer attention stack that share block tables and lengths."""

    def __init__(self, layers, batch, Hq, Hkv, num_phys_blocks, max_blocks, block_tables, seq_lens,
                 sinks=4, window=2048, scale=None, device="cuda", separate_outputs=False, local_only=(),
                 local_tiles=True):
        self.layers, self.batch, self.Hq, self.Hkv = layers, batch, Hq, Hkv
        self.local_only = frozenset(int(l) for l in local_only)
        if any(l < 0 or l >= layers for l in self.local_only):
            raise ValueError("local_only names a layer outside [0, %d)" % layers)
        self.sinks, self.window = sinks, window
        self.scale = 1.0 / math.sqrt(ops.HEAD_DIM) if scale is None else scale
        self.seq_lens = seq_lens
        self.block_tables = block_tables
        self.caches = [ops.PagedKVCache(num_phys_blocks, batch, Hq, Hkv, max_blocks, device=device,
                                        block_tables=block_tables, seq_lens=seq_lens) for _ in range(layers)]
        self.ws = ops.workspace(batch, Hq, device)
        shape = (layers, batch, Hq, ops.HEAD_DIM)
        self.out = torch.zeros(shape, dtype=torch.float32, device=device)
        self.out_full = torch.zeros(shape, dtype=torch.float32, device=device) if separate_outputs else self.out
        self.gate = torch.zeros(batch, dtype=torch.int32, device=device)
        self.qscore = torch.zeros(batch, dtype=torch.float32, device=device)
        # the Local view's tile table, built once per step for every layer (the layers share
        # block tables and lengths); None: every Local launch reads the block table itself
        self.tab = (torch.zeros(ops.local_tiles_bytes(batch, sinks, window, max_blocks) // 4, dtype=torch.int32,
                                device=device) if local_tiles else None)

    def _local(self, l, q, k, v, out, sel=None, sel_value=ops.MODE_LOCAL):
        if self.tab is None:
            ops.oda_decode_local(q, self.caches[l], k, v, self.sinks, self.window, self.scale, sel=sel,
                                 sel_value=sel_value, out=out, ws=self.ws)
        else:
            ops.oda_decode_local_tiles(q, self.caches[l], self.tab, k, v, self.sinks, self.window, self.scale,
                                       sel=sel, sel_value=sel_value, out=out, ws=self.ws)

    def local_pass(self, q, k, v):
        """q: [L][B][Hq][128] fp32, k, v: [L][B][Hkv][128] bf16 (Local candidates). With a
        tile table, the step's Local tiles are listed once, then every layer attends them."""
        if self.tab is not None:
            ops.local_tiles(self.caches[0], self.sinks, self.window, tab=self.tab)
        for l in range(self.layers):
            self._local(l, q[l], k[l], v[l], self.out[l])

    def gate_from_scores(self, scores, theta=0.0):
        ops.oda_gate_scores(scores, theta, out=self.gate)

    def gate_from_recall_head(self, x, W1, b1, w2, b2, theta=0.0):
        ops.oda_recall_score(x, W1, b1, w2, b2, theta, q_out=self.qscore, gate_out=self.gate, ws=self.ws)

    def full_pass(self, q, k, v, gated=True):
        """The recall pass: Full view per layer, Local view for local-only layers."""
        sel = self.gate if gated else None
        for l in range(self.layers):
            if l in self.local_only:  # the table of this step's Local pass, if any, still holds
                self._local(l, q[l], k[l], v[l], self.out_full[l], sel=sel, sel_value=1)
            else:
                ops.oda_decode_full(q[l], self.caches[l], k[l], v[l], self.scale, sel=sel, sel_value=1,
                                    out=self.out_full[l], ws=self.ws)


class RaggedBatch:
    """One attention layer over a ragged batch with per-request views. one_launch: the
    three views in one decode launch (oda_decode_views, after da_gather for the block
    requests); otherwise one selector launch per view."""

    def __init__(self, cache, fallback, keep_mask, sinks=4, window=2048, scale=None, device="cuda",
                 one_launch=True):
        self.one_launch = one_launch
        self.cache = cache
        self.fallback = fallback
        self.keep_mask = keep_mask
        self.sinks, self.window = sinks, window
        self.scale = 1.0 / math.sqrt(ops.HEAD_DIM) if scale is None else scale
        B, mb = cache.batch, cache.max_blocks
        self.ws = ops.workspace(B, cache.num_q_heads, device)
        self.mode = torch.zeros(B, dtype=torch.int32, device=device)
        self.out = torch.zeros((B, cache.num_q_heads, ops.HEAD_DIM), dtype=torch.float32, device=device)
        self.gathered = torch.zeros((B, mb), dtype=torch.int32, device=device)
        self.gathered_cnt = torch.zeros((B, mb), dtype=torch.int32, device=device)
        self.num_kept = torch.zeros(B, dtype=torch.int32, device=device)

    def step(self, q, k, v, scores, theta=0.0):
        """q: [B][Hq][128] fp32; k, v: [B][Hkv][128] bf16; scores: [B] fp32."""
        ops.oda_gate_scores(scores, theta, fallback=self.fallback, out=self.mode)
        if self.one_launch:
            ops.da_gather(self.cache, self.keep_mask, gathered=self.gathered, gathered_cnt=self.gathered_cnt,
                          num_kept=self.num_kept, sel=self.mode, sel_value=ops.MODE_BLOCKS, ws=self.ws)
            ops.oda_decode_views(q, self.cache, self.mode, self.gathered, self.gathered_cnt, self.num_kept, k, v,
                                 self.sinks, self.window, self.scale, out=self.out, ws=self.ws)
            return
        ops.oda_decode_full(q, self.cache, k, v, self.scale, sel=self.mode, sel_value=ops.MODE_FULL,
                            out=self.out, ws=self.ws)
        ops.oda_decode_local(q, self.cache, k, v, self.sinks, self.window, self.scale, sel=self.mode,
                             sel_value=ops.MODE_LOCAL, out=self.out, ws=self.ws)
        ops.da_decode_blocks(q, self.cache, self.keep_mask, k, v, self.scale, sel=self.mode,
                             sel_value=ops.MODE_BLOCKS, out=self.out, gathered=self.gathered,
                             gathered_cnt=self.gathered_cnt, num_kept=self.num_kept, ws=self.ws)


class DAStep:
    """One attention layer driven by Declarative-Attention declarations. By default the
    declaration becomes a keep mask, the mask a gathered list (the rewritten block table)
    and the list is attended; with in_kernel_rewrite the decode kernel derives the kept
    blocks from the declaration itself (da_decode_declared: same result, one launch)."""

    def __init__(self, cache, local_tokens=1024, scale=None, device="cuda", in_kernel_rewrite=False):
        self.cache = cache
        self.in_kernel_rewrite = in_kernel_rewrite
        self.local_tokens = local_tokens
        self.scale = 1.0 / math.sqrt(ops.HEAD_DIM) if scale is None else scale
        B, mb = cache.batch, cache.max_blocks
        self.ws = ops.workspace(B, cache.num_q_heads, device)
        self.mask = torch.zeros((B, (mb + 31) // 32), dtype=torch.int32, device=device)
        self.out = torch.zeros((B, cache.num_q_heads, ops.HEAD_DIM), dtype=torch.float32, device=device)
        self.gathered = torch.zeros((B, mb), dtype=torch.int32, device=device)
        self.gathered_cnt = torch.zeros((B, mb), dtype=torch.int32, device=device)
        self.num_kept = torch.zeros(B, dtype=torch.int32, device=device)

    def step(self, q, k, v, decl):
        if self.in_kernel_rewrite:
            ops.da_decode_declared(q, self.cache, decl, self.local_tokens, k, v, self.scale, out=self.out,
                                   ws=self.ws)
            return
        ops.da_keep_mask(decl, self.cache, self.local_tokens, mask=self.mask)
        ops.da_decode_blocks(q, self.cache, self.mask, k, v, self.scale, out=self.out, gathered=self.gathered,
                             gathered_cnt=self.gathered_cnt, num_kept=self.num_kept, ws=self.ws)


class DATagStep(DAStep):
    """One attention layer whose declarations come from the generated tokens: each step
    the input token advances the per-request parser (mode tags, named segments), which
    writes the step's declaration and keep mask, then the kept blocks are attended."""

    def __init__(self, cache, tags, output_begin, segments=None, local_tokens=1024, scale=None, device="cuda",
                 in_kernel_rewrite=False):
        super().__init__(cache, local_tokens, scale, device, in_kernel_rewrite)
        B = cache.batch
        self.tags = tuple(int(x) for x in tags)
        self.output_begin = output_begin
        self.segments = segments
        self.state = torch.zeros((B, 4), dtype=torch.int32, device=device)  # {global, 0, 0, no focus pending}
        self.decl = torch.zeros((B, 4), dtype=torch.int32, device=device)

    def step(self, q, k, v, tokens):
        ops.da_declare(tokens, self.state, self.output_begin, self.cache, self.tags, segments=self.segments,
                       local_tokens=self.local_tokens, decl=self.decl, mask=self.mask,
                       with_mask=not self.in_kernel_rewrite)
        if self.in_kernel_rewrite:
            ops.da_decode_declared(q, self.cache, self.decl, self.local_tokens, k, v, self.scale, out=self.out,
                                   ws=self.ws)
            return
        ops.da_decode_blocks(q, self.cache, self.mask, k, v, self.scale, out=self.out, gathered=self.gathered,
                             gathered_cnt=self.gathered_cnt, num_kept=self.num_kept, ws=self.ws)


class HostRoutedStep:
    """One decode step as graphs with the recall branch taken on the host.

    first: the launches up to and including the gate (feed, Local pass, gate);
    recall: the gated recall pass (and whatever follows it on a recall step);
    skip: optional launches that replace `recall` on a step without a recall.
    gate: the int32 gate tensor that `first` writes, one entry per request.
    replay() returns whether the recall graph ran.
    """

    def __init__(self, first, recall, gate, skip=None):
        self.first = capture_graph(first)
        self.recall = capture_graph(recall)
        self.skip = capture_graph(skip) if skip is not None else None
        self.gate = gate
        self.host_gate = torch.zeros(gate.numel(), dtype=torch.int32, pin_memory=True)
        self.host_view = self.host_gate.numpy()
        self.read = torch.cuda.Event()

    def replay(self):
        self.first.replay()
        self.host_gate.copy_(self.gate, non_blocking=True)
        self.read.record()
        self.read.synchronize()
        recalled = bool(np.any(self.host_view))
        if recalled:
            self.recall.replay()
        elif self.skip is not None:
            self.skip.replay()
        return recalled


def capture_graph(fn):
    """Capture the launches made by fn() into a HIP graph (replayed with .replay())."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    return g
