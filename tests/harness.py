"""Step-by-step runs of the synthetic workloads on the GPU, mirrored in the fp64 oracle.

Each run drives the library through ``sparse_kv_recall_amd.stack`` (optionally as a
captured HIP graph, the configuration bench.py times) and, after every step, checks
the GPU results against the oracle on the same seeded inputs:

* recall decisions and gathered block lists bit-exact (decisions with |q - theta| < 1e-4
  are excluded; the oracle then adopts the GPU's decision so the histories stay equal);
* attention outputs within max-abs 2e-3 and row-relative 1e-2;
* committed KV slots bit-exact at the end.

The host mirrors hold the logical K/V of the checked layers / requests; everything
else lives only on the GPU.
"""

import math

import numpy as np
import torch

import oracle
from oracle import attention, gather, keysets
from sparse_kv_recall_amd import ops
from sparse_kv_recall_amd.stack import DAStep, HostRoutedStep, ODAStack, RaggedBatch, capture_graph
from synth import device as sdev
from synth import rng
from synth.workloads import C_KHIST, C_VHIST
from tests.helpers import bf16_tensor_to_bits, check_close

SCALE = 1.0 / math.sqrt(128.0)
BAND = 1e-4


class Report:
    def __init__(self):
        self.max_abs = 0.0
        self.max_row_rel = 0.0
        self.checked_outputs = 0
        self.decisions = 0
        self.decisions_in_band = 0
        self.recalls = 0
        self.commit_layers = 0

    def add(self, got, ref, what):
        a, r = check_close(got, ref, what=what)
        self.max_abs = max(self.max_abs, a)
        self.max_row_rel = max(self.max_row_rel, r)
        self.checked_outputs += 1


def _fill_history(cache, wl, unit, H0, request=0):
    stage_k = torch.empty((H0, wl.Hkv, 128), dtype=torch.bfloat16, device="cuda")
    stage_v = torch.empty_like(stage_k)
    sdev.fill_normal_(stage_k, wl.key(C_KHIST, unit), 0)
    sdev.fill_normal_(stage_v, wl.key(C_VHIST, unit), 0)
    ops.kv_write(cache, request, 0, stage_k, stage_v)
    torch.cuda.synchronize()


def _mirror(wl, unit, H0, steps):
    k = np.zeros((H0 + steps, wl.Hkv, 128), np.uint16)
    v = np.zeros_like(k)
    k[:H0] = wl.hist_bits("k", unit, 0, H0)
    v[:H0] = wl.hist_bits("v", unit, 0, H0)
    return k, v


class OdaStackRun:
    """ODA stack (Local every step, on-device gate, gated Full) with host mirrors of
    ``check_layers``."""

    def __init__(self, wl, check_layers, steps=None, use_graph=True, local_only=(), same_candidates=False,
                 host_routed=False):
        self.wl = wl
        self.steps = wl.steps if steps is None else steps
        self.check_layers = list(check_layers)
        self.use_graph = use_graph
        self.local_only = frozenset(local_only)
        # same_candidates: the recall pass is fed the Local pass's q / k / v (what a model
        # computes when no earlier layer's result changed), instead of its own stream
        self.rpass = 0 if same_candidates else 1
        H0 = int(wl.H0[0])
        bt = torch.as_tensor(wl.block_tables, device="cuda")
        seq = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.stack = ODAStack(wl.layers, 1, wl.Hq, wl.Hkv, wl.num_phys_blocks, wl.max_blocks, bt, seq,
                              sinks=wl.sinks, window=wl.window, separate_outputs=True,
                              local_only=self.local_only)
        for l in range(wl.layers):
            _fill_history(self.stack.caches[l], wl, l, H0)
        self.recall_head = wl.x_dim > 0
        self.feeder = sdev.Feeder(wl, seq, with_x=self.recall_head, with_scores=not self.recall_head)
        if self.recall_head:
            W1, b1, w2, b2 = wl.recall_weights()
            self.host_w = (W1, b1, w2, b2)
            self.dev_w = tuple(torch.as_tensor(a, device="cuda") for a in (W1, b1, w2, b2))
        self.mirror = {l: _mirror(wl, l, H0, self.steps) for l in self.check_layers}
        if host_routed:  # two graphs, the recall pass replayed on the host's reading of the gate
            self.graph = HostRoutedStep(self._first, self._recall, self.stack.gate)
        else:
            self.graph = capture_graph(self._step) if use_graph else None

    def _first(self):
        f, s = self.feeder, self.stack
        f.step()
        s.local_pass(f.q[:, 0], f.k[:, 0], f.v[:, 0])
        if self.recall_head:
            s.gate_from_recall_head(f.x, *self.dev_w, theta=self.wl.theta)
        else:
            s.gate_from_scores(f.scores, self.wl.theta)

    def _recall(self):
        f, p = self.feeder, self.rpass
        self.stack.full_pass(f.q[:, p], f.k[:, p], f.v[:, p], gated=True)

    def _step(self):
        self._first()
        self._recall()

    def run(self, full_check_steps=None, check_feed_steps=(0,), commit_all_layers=False, full_sample=None):
        """full_check_steps: recall steps whose Full outputs are checked (None: all);
        commit_all_layers: also check the committed slots of every layer (not only the
        mirrored ones) against the selected pass's candidates regenerated from the
        seeded streams; full_sample: a seeded numpy Generator, with which every other
        recall step checks the query heads of one KV head of one mirrored layer (drawn
        from it), the oracle computing that head group alone."""
        wl, rep = self.wl, Report()
        H0 = int(wl.H0[0])
        gates = []
        for t in range(self.steps):
            ran = self.graph.replay() if self.graph is not None else self._step()
            torch.cuda.synchronize()
            n = H0 + t + 1
            assert int(self.stack.seq_lens[0].item()) == n
            gpu_gate = int(self.stack.gate[0].item())
            if isinstance(self.graph, HostRoutedStep):  # the recall graph ran exactly on gated steps
                assert ran == bool(gpu_gate), (t, ran, gpu_gate)
            if t in check_feed_steps:  # the device feed reproduces the host streams bit for bit
                for l in self.check_layers:
                    assert np.array_equal(self.feeder.q[l, 1, 0].cpu().numpy(), wl.cand_q(t, l, 1, 0))
                    k1, _ = wl.cand_kv(t, l, 1, 0)
                    assert np.array_equal(bf16_tensor_to_bits(self.feeder.k[l, 1, 0]), k1)
            # decision
            if self.recall_head:
                x = wl.recall_x(t, 0)
                q_ref = oracle.recall.recall_score(x, *self.host_w)
                q_gpu = float(self.stack.qscore[0].item())
                assert abs(q_gpu - q_ref) <= 1e-4 * max(1.0, abs(q_ref)), (t, q_gpu, q_ref)
                if abs(q_ref - wl.theta) < BAND:
                    rep.decisions_in_band += 1
                    gate = bool(gpu_gate)
                else:
                    gate = oracle.recall.gate(q_ref, wl.theta)
                    assert gate == bool(gpu_gate), (t, q_ref, gpu_gate)
            else:
                gate = oracle.recall.gate(float(wl.score(t, 0)), wl.theta)
                assert gate == bool(gpu_gate), t
            rep.decisions += 1
            rep.recalls += int(gate)
            gates.append(bool(gate))
            out_l = self.stack.out.cpu().numpy() if self.check_layers else None
            out_f = self.stack.out_full.cpu().numpy() if (gate and self.check_layers) else None
            sampled = None  # (layer, KV head) whose Full rows this recall step checks
            if gate and full_sample is not None and full_check_steps is not None and t not in full_check_steps:
                sampled = (self.check_layers[int(full_sample.integers(len(self.check_layers)))],
                           int(full_sample.integers(wl.Hkv)))
            for l in self.check_layers:
                hk, hv = self.mirror[l]
                qL = wl.cand_q(t, l, 0, 0)
                kL, vL = wl.cand_kv(t, l, 0, 0)
                oL = oracle.oda.local_pass(qL, kL, vL, hk, hv, n, SCALE, wl.sinks, wl.window)
                rep.add(out_l[l, 0], oL, "local t=%d layer=%d" % (t, l))
                if gate:
                    qF = wl.cand_q(t, l, self.rpass, 0)
                    kF, vF = wl.cand_kv(t, l, self.rpass, 0)
                    if full_check_steps is None or t in full_check_steps:
                        oF = oracle.oda.recall_pass(qF, kF, vF, hk, hv, n, SCALE, l in self.local_only,
                                                    wl.sinks, wl.window)
                        rep.add(out_f[l, 0], oF, "recall t=%d layer=%d" % (t, l))
                    else:
                        oracle.oda.commit(hk, hv, n, kF, vF)
                        if sampled is not None and l == sampled[0]:
                            G, g = wl.Hq // wl.Hkv, sampled[1]
                            keys = (keysets.local_keys(n, wl.sinks, wl.window) if l in self.local_only
                                    else keysets.full_keys(n))
                            oF = attention.attend(qF[g * G:(g + 1) * G], hk[:, g:g + 1], hv[:, g:g + 1], keys, SCALE)
                            rep.add(out_f[l, 0, g * G:(g + 1) * G], oF, "recall t=%d layer=%d kv head %d" % (t, l, g))
                    if self.rpass == 0 and l in self.local_only:
                        # the same kernel on the same inputs: the recall result is the Local one
                        assert np.array_equal(out_f[l, 0], out_l[l, 0]), (t, l)
        # committed slots hold the selected candidates, bit for bit
        for l in self.check_layers:
            hk, hv = self.mirror[l]
            k, v = ops.kv_read(self.stack.caches[l], 0, H0, self.steps)
            assert np.array_equal(bf16_tensor_to_bits(k), hk[H0:H0 + self.steps]), l
            assert np.array_equal(bf16_tensor_to_bits(v), hv[H0:H0 + self.steps]), l
        if commit_all_layers:
            for l in range(wl.layers):
                k, v = ops.kv_read(self.stack.caches[l], 0, H0, self.steps)
                kb, vb = bf16_tensor_to_bits(k), bf16_tensor_to_bits(v)
                for t in range(self.steps):
                    ke, ve = wl.cand_kv(t, l, self.rpass if gates[t] else 0, 0)
                    assert np.array_equal(kb[t], ke) and np.array_equal(vb[t], ve), (l, t, gates[t])
            rep.commit_layers = wl.layers
        return rep


class DaRun:
    """Declarative-Attention workload: per step a declared mode -> keep mask -> gathered
    block list -> attention over the kept blocks (with the current token committed)."""

    def __init__(self, wl, steps=None, use_graph=True, in_kernel_rewrite=False):
        self.wl = wl
        self.steps = wl.steps if steps is None else steps
        self.in_kernel_rewrite = in_kernel_rewrite
        H0 = int(wl.H0[0])
        bt = torch.as_tensor(wl.block_tables, device="cuda")
        seq = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.cache = ops.PagedKVCache(wl.num_phys_blocks, 1, wl.Hq, wl.Hkv, wl.max_blocks, block_tables=bt,
                                      seq_lens=seq)
        self.cache.k_pool.view(torch.int16).fill_(0x7FC0)  # unwritten slots are NaN
        self.cache.v_pool.view(torch.int16).fill_(0x7FC0)
        _fill_history(self.cache, wl, 0, H0)
        self.da = DAStep(self.cache, wl.da_local_tokens, in_kernel_rewrite=in_kernel_rewrite)
        self.feeder = sdev.Feeder(wl, seq, with_decl=True)
        self.mirror = _mirror(wl, 0, H0, self.steps)
        self.graph = capture_graph(self._step) if use_graph else None

    def _step(self):
        f = self.feeder
        f.step()
        self.da.step(f.q[0, 0], f.k[0, 0], f.v[0, 0], f.decl)

    def run(self, check_steps=None):
        wl, rep = self.wl, Report()
        H0 = int(wl.H0[0])
        hk, hv = self.mirror
        pb = wl.extra["prompt_blocks"]
        for t in range(self.steps):
            self.graph.replay() if self.graph is not None else self._step()
            torch.cuda.synchronize()
            n = H0 + t + 1
            mode, f0, f1, ob = (int(x) for x in wl.decl[t, 0])
            assert ob == pb
            kept = gather.da_mode_blocks(mode, n, f0, f1, ob, local_tokens=wl.da_local_tokens)
            if not self.in_kernel_rewrite:  # the rewritten block table is materialised
                phys, cnt = gather.gather_blocks(wl.block_tables[0], kept, n)
                num = int(self.da.num_kept[0].item())
                assert num == len(phys), t
                assert np.array_equal(self.da.gathered[0, :num].cpu().numpy(), phys), t
                assert np.array_equal(self.da.gathered_cnt[0, :num].cpu().numpy(), cnt), t
            q = wl.cand_q(t, 0, 0, 0)
            kN, vN = wl.cand_kv(t, 0, 0, 0)
            if check_steps is None or t in check_steps:
                o = oracle.oda.blocks_pass(q, kN, vN, hk, hv, n, kept, SCALE)
                rep.add(self.da.out[0].cpu().numpy(), o, "da t=%d mode=%d" % (t, mode))
            else:
                oracle.oda.commit(hk, hv, n, kN, vN)
            rep.decisions += 1
        k, v = ops.kv_read(self.cache, 0, H0, self.steps)
        assert np.array_equal(bf16_tensor_to_bits(k), hk[H0:H0 + self.steps])
        assert np.array_equal(bf16_tensor_to_bits(v), hv[H0:H0 + self.steps])
        return rep


class DaTagsRun:
    """Declarative-Attention layer driven by a token stream: per step the input token
    advances the device parser (checked against the oracle parser: state and
    declaration bit for bit), then keep mask -> gathered list -> attention."""

    def __init__(self, wl, steps=None, use_graph=True, in_kernel_rewrite=False):
        from sparse_kv_recall_amd.stack import DATagStep
        self.wl = wl
        self.steps = wl.steps if steps is None else steps
        self.in_kernel_rewrite = in_kernel_rewrite
        H0 = int(wl.H0[0])
        bt = torch.as_tensor(wl.block_tables, device="cuda")
        seq = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.cache = ops.PagedKVCache(wl.num_phys_blocks, 1, wl.Hq, wl.Hkv, wl.max_blocks, block_tables=bt,
                                      seq_lens=seq)
        self.cache.k_pool.view(torch.int16).fill_(0x7FC0)  # unwritten slots are NaN
        self.cache.v_pool.view(torch.int16).fill_(0x7FC0)
        _fill_history(self.cache, wl, 0, H0)
        self.da = DATagStep(self.cache, wl.da_tags, torch.as_tensor(wl.output_begin, device="cuda"),
                            segments=torch.as_tensor(wl.segments, device="cuda"), local_tokens=wl.da_local_tokens,
                            in_kernel_rewrite=in_kernel_rewrite)
        self.feeder = sdev.Feeder(wl, seq, with_tokens=True)
        self.mirror = _mirror(wl, 0, H0, self.steps)
        self.graph = capture_graph(self._step) if use_graph else None

    def _step(self):
        f = self.feeder
        f.step()
        self.da.step(f.q[0, 0], f.k[0, 0], f.v[0, 0], f.tokens)

    def run(self, check_steps=None):
        wl, rep = self.wl, Report()
        H0 = int(wl.H0[0])
        hk, hv = self.mirror
        rows, states = oracle.declare.parse_declarations(wl.tokens[:self.steps, 0], wl.da_tags,
                                                          wl.segments[0].tolist(), int(wl.output_begin[0]))
        for t in range(self.steps):
            self.graph.replay() if self.graph is not None else self._step()
            torch.cuda.synchronize()
            n = H0 + t + 1
            assert tuple(int(x) for x in self.da.state[0].cpu()) == states[t], t
            assert tuple(int(x) for x in self.da.decl[0].cpu()) == rows[t], t
            mode, fb, fe, ob = rows[t]
            kept = gather.da_mode_blocks(mode, n, fb, fe, ob, local_tokens=wl.da_local_tokens)
            if not self.in_kernel_rewrite:  # keep mask and rewritten block table are materialised
                words = self.da.mask[0].cpu().numpy().view(np.uint32)
                assert gather.mask_to_blocks(words, n) == kept, t
                phys, cnt = gather.gather_blocks(wl.block_tables[0], kept, n)
                num = int(self.da.num_kept[0].item())
                assert num == len(phys), t
                assert np.array_equal(self.da.gathered[0, :num].cpu().numpy(), phys), t
                assert np.array_equal(self.da.gathered_cnt[0, :num].cpu().numpy(), cnt), t
            q = wl.cand_q(t, 0, 0, 0)
            kN, vN = wl.cand_kv(t, 0, 0, 0)
            if check_steps is None or t in check_steps:
                o = oracle.oda.blocks_pass(q, kN, vN, hk, hv, n, kept, SCALE)
                rep.add(self.da.out[0].cpu().numpy(), o, "da-tags t=%d mode=%d" % (t, mode))
            else:
                oracle.oda.commit(hk, hv, n, kN, vN)
            rep.decisions += 1
            rep.recalls += int(mode == gather.FOCUS)
        k, v = ops.kv_read(self.cache, 0, H0, self.steps)
        assert np.array_equal(bf16_tensor_to_bits(k), hk[H0:H0 + self.steps])
        assert np.array_equal(bf16_tensor_to_bits(v), hv[H0:H0 + self.steps])
        return rep


class RaggedRun:
    """Ragged batch: per step each request takes Full (score > theta) or its fallback
    view (Local, or its fixed keep-list); host mirrors for ``check_requests``."""

    def __init__(self, wl, check_requests, steps=None, use_graph=True, one_launch=True):
        self.wl = wl
        self.steps = wl.steps if steps is None else steps
        self.check = list(check_requests)
        bt = torch.as_tensor(wl.block_tables, device="cuda")
        seq = torch.zeros(wl.batch, dtype=torch.int32, device="cuda")
        self.cache = ops.PagedKVCache(wl.num_phys_blocks, wl.batch, wl.Hq, wl.Hkv, wl.max_blocks,
                                      block_tables=bt, seq_lens=seq)
        for r in range(wl.batch):
            _fill_history(self.cache, wl, r, int(wl.H0[r]), request=r)
        self.rb = RaggedBatch(self.cache, torch.as_tensor(wl.fallback, device="cuda"),
                              torch.as_tensor(wl.keep_mask.view(np.int32), device="cuda"),
                              sinks=wl.sinks, window=wl.window, one_launch=one_launch)
        self.feeder = sdev.Feeder(wl, seq, with_scores=True)
        self.mirror = {r: _mirror(wl, r, int(wl.H0[r]), self.steps) for r in self.check}
        self.graph = capture_graph(self._step) if use_graph else None

    def _step(self):
        f = self.feeder
        f.step()
        self.rb.step(f.q[0, 0], f.k[0, 0], f.v[0, 0], f.scores, self.wl.theta)

    def run(self, check_steps=None, commit_all_requests=False):
        """check_steps: steps whose outputs of the mirrored requests are checked (None:
        all); commit_all_requests: also check every request's committed slots (each view
        commits the request's candidate) against the candidates regenerated from the
        seeded streams."""
        wl, rep = self.wl, Report()
        for t in range(self.steps):
            self.graph.replay() if self.graph is not None else self._step()
            torch.cuda.synchronize()
            mode_gpu = self.rb.mode.cpu().numpy()
            scores = wl.scores_all()[t]
            out = self.rb.out.cpu().numpy() if (check_steps is None or t in check_steps) else None
            for r in range(wl.batch):
                s = float(scores[r])
                if abs(s - wl.theta) < BAND:
                    rep.decisions_in_band += 1
                    mode = int(mode_gpu[r])
                else:
                    mode = oracle.oda.request_mode(s, wl.theta, int(wl.fallback[r]))
                    assert mode == int(mode_gpu[r]), (t, r)
                rep.decisions += 1
                rep.recalls += int(mode == oracle.oda.MODE_FULL)
                if r not in self.mirror:
                    continue
                n = int(wl.H0[r]) + t + 1
                hk, hv = self.mirror[r]
                q = wl.cand_q(t, 0, 0, r)
                kN, vN = wl.cand_kv(t, 0, 0, r)
                if mode == oracle.oda.MODE_FULL:
                    keys = keysets.full_keys(n)
                elif mode == oracle.oda.MODE_LOCAL:
                    keys = keysets.local_keys(n, wl.sinks, wl.window)
                else:
                    kept = gather.mask_to_blocks(wl.keep_mask[r], n)
                    keys = keysets.block_keys(n, kept)
                    phys, cnt = gather.gather_blocks(wl.block_tables[r], kept, n)
                    num = int(self.rb.num_kept[r].item())
                    assert num == len(phys)
                    assert np.array_equal(self.rb.gathered[r, :num].cpu().numpy(), phys)
                    assert np.array_equal(self.rb.gathered_cnt[r, :num].cpu().numpy(), cnt)
                oracle.oda.commit(hk, hv, n, kN, vN)
                if out is not None:
                    o = attention.attend(q, hk, hv, keys, SCALE)
                    rep.add(out[r], o, "ragged t=%d r=%d mode=%d" % (t, r, mode))
        for r in self.check:
            H0 = int(wl.H0[r])
            hk, hv = self.mirror[r]
            k, v = ops.kv_read(self.cache, r, H0, self.steps)
            assert np.array_equal(bf16_tensor_to_bits(k), hk[H0:H0 + self.steps]), r
            assert np.array_equal(bf16_tensor_to_bits(v), hv[H0:H0 + self.steps]), r
        if commit_all_requests:
            for r in range(wl.batch):
                k, v = ops.kv_read(self.cache, r, int(wl.H0[r]), self.steps)
                kb, vb = bf16_tensor_to_bits(k), bf16_tensor_to_bits(v)
                for t in range(self.steps):
                    ke, ve = wl.cand_kv(t, 0, 0, r)
                    assert np.array_equal(kb[t], ke) and np.array_equal(vb[t], ve), (r, t)
            rep.commit_layers = wl.batch
        return rep


class DecoderRun:
    """Weight-bearing ODA steps (Local pass through every layer, recall head on the real
    Local hidden state, gated recall pass, select) against the fp64 decoder oracle."""

    def __init__(self, wl, local_only=(), fuse_qk=True):
        from sparse_kv_recall_amd.model import DecoderShape, ODADecoder
        self.wl = wl
        L, Hkv = wl.layers, wl.kv_heads
        mb = wl.max_blocks
        bt = torch.arange(mb, dtype=torch.int32, device="cuda")[None]
        self.seq = torch.full((1,), wl.H0, dtype=torch.int32, device="cuda")
        self.caches = [ops.PagedKVCache(mb, 1, wl.q_heads, Hkv, mb, block_tables=bt, seq_lens=self.seq)
                       for _ in range(L)]
        self.hist = []
        for l, c in enumerate(self.caches):
            k = np.zeros((wl.H0 + wl.steps, Hkv, 128), np.uint16)
            v = np.zeros_like(k)
            k[:wl.H0] = wl.hist_bits("k", l, 0, wl.H0)
            v[:wl.H0] = wl.hist_bits("v", l, 0, wl.H0)
            ops.kv_write(c, 0, 0, torch.as_tensor(k[:wl.H0].view(np.int16), device="cuda").view(torch.bfloat16),
                         torch.as_tensor(v[:wl.H0].view(np.int16), device="cuda").view(torch.bfloat16))
            self.hist.append((k, v))
        shape = DecoderShape(L, wl.hidden, wl.q_heads, Hkv, wl.intermediate, wl.vocab, wl.recall_hidden, wl.eps,
                             wl.rope_base)
        self.model = ODADecoder(shape, wl.device_weights(), self.caches, wl.sinks, wl.window,
                                local_only=local_only, fuse_qk=fuse_qk)
        self.local_only = frozenset(local_only)
        self.oracle = oracle.decoder.Decoder(
            oracle.decoder.DecoderShape(L, wl.hidden, wl.q_heads, Hkv, wl.intermediate, wl.vocab, wl.recall_hidden,
                                        eps=wl.eps, rope_base=wl.rope_base), wl.host_weights())

    def run(self):
        wl, rep, m = self.wl, Report(), self.model
        h_prev = np.zeros(wl.hidden)
        n_bad, n_all = 0, 0
        for t in range(wl.steps):
            n = wl.H0 + t + 1
            tok = int(wl.tokens[t])
            m.token.fill_(tok)
            self.seq.fill_(n)
            m.step(wl.theta)
            torch.cuda.synchronize()
            q_gpu = float(m.qscore[0].item())
            g_gpu = bool(m.gate[0].item())

            def decide(q):
                if abs(q - wl.theta) < BAND:
                    rep.decisions_in_band += 1
                    return g_gpu
                return oracle.recall.gate(q, wl.theta)

            if self.local_only:
                hs, g, q_ref, hL = self._oracle_step_local_only(tok, h_prev, n, decide)
            else:
                hs, g, q_ref, hL = self.oracle.oda_step(tok, h_prev, self.hist, n, wl.theta, decide=decide,
                                                        sinks=wl.sinks, window=wl.window)
            assert abs(q_gpu - q_ref) <= 1e-3 * max(1.0, abs(q_ref)), (t, q_gpu, q_ref)
            assert g == g_gpu, (t, q_gpu, q_ref)
            rep.decisions += 1
            rep.recalls += int(g)
            rep.add(m.h_local_final.cpu().numpy()[None], hL[None], "h_local t=%d" % t)
            rep.add(m.h_prev.cpu().numpy()[None], hs[None], "h_selected t=%d" % t)
            for l in range(wl.layers):  # committed candidates: bf16 of nearly equal values
                k, v = ops.kv_read(self.caches[l], 0, n - 1, 1)
                for got, ref in ((bf16_tensor_to_bits(k)[0], self.hist[l][0][n - 1]),
                                 (bf16_tensor_to_bits(v)[0], self.hist[l][1][n - 1])):
                    a, b = oracle.bf16_bits_to_f64(got), oracle.bf16_bits_to_f64(ref)
                    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(a), np.abs(b)) + 1e-30), (t, l)
                    n_bad += int((got != ref).sum())
                    n_all += got.size
            h_prev = hs
        rep.commit_mismatch_frac = n_bad / max(1, n_all)
        assert rep.commit_mismatch_frac < 0.01, rep.commit_mismatch_frac
        return rep

    def _oracle_step_local_only(self, tok, h_prev, n, decide):
        # per-layer access control in the recall pass (local-only layers keep the Local view)
        dec, wl = self.oracle, self.wl
        hL = dec.forward(tok, self.hist, n, False, sinks=wl.sinks, window=wl.window)
        x = oracle.recall.concat_inputs(h_prev, dec.w["emb"][tok], hL)
        q_t = oracle.recall.recall_score(x, dec.w["W1"], dec.w["b1"], dec.w["w2"], dec.w["b2"])
        if not decide(q_t):
            return hL, False, q_t, hL
        scale = 1.0 / math.sqrt(128)
        h = dec.w["emb"][tok].copy()
        for l in range(wl.layers):
            full = l not in self.local_only
            h = dec.layer(l, h, self.hist[l][0], self.hist[l][1], n, full, scale, wl.sinks, wl.window)
        return oracle.decoder.rms_norm(h, dec.w["g_final"], wl.eps), True, q_t, hL
