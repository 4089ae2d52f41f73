"""Seeded synthetic workloads: shapes, value streams and per-step schedules.

Five workloads, each a stand-in for a setting the pages measure on (no dataset,
tokenizer or trained weight is used; only shapes, sizes and value
distributions are kept):

1. ``oda_small``  1 layer, 8 query / 2 KV heads, history 4096, 64 steps; Local
   every step, Full on a seeded Bernoulli(0.4) step.
2. ``oda_stack16k``  28 layers, 16 / 8 heads, history 16384, 256 steps; the
   recall head is a 6144 -> 512 -> 1 MLP with N(0, 0.02^2) weights, zero
   biases and N(0, 1) hidden states; theta = 0.
3. ``oda_stack128k``  36 layers, 32 / 8 heads, history 131072 growing by 1024
   steps, Full on exactly 128 seeded steps (12.5 %): one at a seeded offset in
   every aligned run of 8 steps; block table = identity.
4. ``da_32k``  1 layer, 32 / 8 heads, context 32768 (1984 prompt blocks + 64
   blocks of earlier model output) growing by 512 steps; per step a seeded
   declared mode (global / focus on 128 blocks / local 1024 positions); the
   physical placement is a seeded permutation of a 2080-block pool.
5. ``ragged32``  32 requests, 32 / 8 heads, lengths log-uniform in
   [4096, 131072], shared permuted pool, 256 steps; per step a request takes
   Full when its N(0,1) score > 0, else its seeded fallback (Local, or a fixed
   keep-list of 5-20 % of its blocks plus every block from the one holding
   position L_r onwards).

A sixth, ``da_tags_32k``, is ``da_32k``'s shape with the declarations parsed from
a seeded token stream (mode tags, 16 named segments of the prompt) instead of
drawn per step.

Conventions: history positions 0 .. H0-1 are synthetic; at step t (0-based)
the request has n = H0 + t + 1 visible positions and the current token sits at
position H0 + t. Large arrays come from ``synth.rng`` streams keyed by
(workload id, component, unit) with these element-index layouts:

* history K / V of a unit (layer or request): index (pos * Hkv + g) * 128 + d
* q candidates:  ((((t * L + l) * P + p) * B + b) * Hq + h) * 128 + d
* k / v candidates: ((((t * L + l) * P + p) * B + b) * Hkv + g) * 128 + d
  with p = 0 (Local) or 1 (Full); at layer 0 both passes use p = 0, because the
  two passes start from the same input there.
* recall input x: (t * B + b) * x_dim + i;  scores: t * B + b
"""

import math
from dataclasses import dataclass, field

import numpy as np

from . import rng

D = 128
BLOCK = 16

# component ids of the stream keys
C_KHIST, C_VHIST, C_Q, C_K, C_V, C_X, C_W1, C_W2, C_SCORE = 1, 2, 3, 4, 5, 6, 7, 8, 9
C_SCHED, C_PERM, C_LEN, C_FALLBACK, C_KEEP, C_MODE, C_TOKENS, C_SEGMENTS = 20, 21, 22, 23, 24, 25, 26, 27

# token ids of the declaration tags in the synthetic vocabulary
TAG_GLOBAL, TAG_FOCUS, TAG_LOCAL, TAG_SEGMENT_BASE = 5, 6, 7, 100

# per-request views of a ragged batch (same numbers as the C header)
MODE_LOCAL, MODE_FULL, MODE_BLOCKS = 0, 1, 2
DA_GLOBAL, DA_FOCUS, DA_LOCAL = 0, 1, 2


def np_rng(*ids):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(i) for i in ids])))


@dataclass
class Workload:
    wid: int
    name: str
    layers: int
    batch: int
    Hq: int
    Hkv: int
    steps: int
    passes: int                 # 2 for the ODA stacks (Local + Full candidates), 1 otherwise
    H0: np.ndarray              # [batch] history length per request
    sinks: int = 4
    window: int = 2048
    theta: float = 0.0
    x_dim: int = 0              # recall-head input width (0: no recall head)
    hidden: int = 0
    block_tables: np.ndarray = None   # [batch][max_blocks] int32
    num_phys_blocks: int = 0
    sched_scores: np.ndarray = None   # [steps][batch] float32 (+1/-1) or None
    decl: np.ndarray = None           # [steps][batch][4] int32 (DA workloads)
    da_local_tokens: int = 1024
    fallback: np.ndarray = None       # [batch] int32 (ragged batch)
    keep_mask: np.ndarray = None      # [batch][words] uint32 fixed keep-lists (ragged batch)
    tokens: np.ndarray = None         # [steps][batch] int32 input token per step (declaration stream)
    segments: np.ndarray = None       # [batch][S][2] int32 named context segments [begin, end)
    output_begin: np.ndarray = None   # [batch] int32 first logical block of the model's output
    da_tags: tuple = None             # (global, focus, local, segment_base) token ids
    extra: dict = field(default_factory=dict)

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def max_blocks(self):
        return self.block_tables.shape[1]

    @property
    def mask_words(self):
        return (self.max_blocks + 31) // 32

    def n_at(self, t):
        return self.H0 + t + 1

    # ---- stream keys
    def key(self, comp, unit=0):
        return rng.mix_key(self.wid, comp, unit)

    # ---- history
    def hist_bits(self, kind, unit, start, count):
        """bf16 bits [count][Hkv][128] of history positions start..start+count-1 of a
        unit (layer for stacks, request for batches); kind 'k' or 'v'."""
        comp = C_KHIST if kind == "k" else C_VHIST
        e = self.Hkv * D
        flat = rng.normal_bf16(self.key(comp, unit), start * e, count * e, rng.unit_scale())
        return flat.reshape(count, self.Hkv, D)

    # ---- per-step candidates
    def _cand_index(self, t, layer, p, b, heads):
        pe = 0 if layer == 0 else p
        return ((((t * self.layers + layer) * self.passes + pe) * self.batch + b) * heads) * D

    def cand_q(self, t, layer, p, b):
        i0 = self._cand_index(t, layer, p, b, self.Hq)
        return rng.normal_f32(self.key(C_Q), i0, self.Hq * D, rng.unit_scale()).reshape(self.Hq, D)

    def cand_kv(self, t, layer, p, b):
        i0 = self._cand_index(t, layer, p, b, self.Hkv)
        k = rng.normal_bf16(self.key(C_K), i0, self.Hkv * D, rng.unit_scale()).reshape(self.Hkv, D)
        v = rng.normal_bf16(self.key(C_V), i0, self.Hkv * D, rng.unit_scale()).reshape(self.Hkv, D)
        return k, v

    # ---- recall head (x_dim > 0)
    def recall_x(self, t, b):
        return rng.normal_f32(self.key(C_X), (t * self.batch + b) * self.x_dim, self.x_dim, rng.unit_scale())

    def recall_weights(self):
        W1 = rng.normal_f32(self.key(C_W1), 0, self.hidden * self.x_dim, rng.unit_scale(0.02))
        w2 = rng.normal_f32(self.key(C_W2), 0, self.hidden, rng.unit_scale(0.02))
        return (W1.reshape(self.hidden, self.x_dim), np.zeros(self.hidden, np.float32), w2,
                np.zeros(1, np.float32))

    # ---- scores of a ragged batch (no recall head): N(0,1) per request per step
    def score(self, t, b):
        if self.sched_scores is not None:
            return np.float32(self.sched_scores[t, b])
        return rng.normal_f32(self.key(C_SCORE), t * self.batch + b, 1, rng.unit_scale())[0]

    def scores_all(self):
        if self.sched_scores is not None:
            return self.sched_scores.astype(np.float32)
        flat = rng.normal_f32(self.key(C_SCORE), 0, self.steps * self.batch, rng.unit_scale())
        return flat.reshape(self.steps, self.batch)


def _blocks_for(n):
    return (n + BLOCK - 1) // BLOCK


def oda_small(steps=64, H0=4096):
    wid = 1
    g = np_rng(wid, C_SCHED)
    recall = g.random(steps) < 0.4
    mb = _blocks_for(H0 + steps)
    return Workload(wid, "oda_small", layers=1, batch=1, Hq=8, Hkv=2, steps=steps, passes=2,
                    H0=np.array([H0], np.int64),
                    block_tables=np.arange(mb, dtype=np.int32)[None, :], num_phys_blocks=mb,
                    sched_scores=np.where(recall, 1.0, -1.0).astype(np.float32)[:, None])


def oda_stack16k(steps=256, H0=16384, layers=28):
    wid = 2
    mb = _blocks_for(H0 + steps)
    return Workload(wid, "oda_stack16k", layers=layers, batch=1, Hq=16, Hkv=8, steps=steps, passes=2,
                    H0=np.array([H0], np.int64), x_dim=3 * 2048, hidden=512,
                    block_tables=np.arange(mb, dtype=np.int32)[None, :], num_phys_blocks=mb)


def oda_stack128k(steps=1024, H0=131072, layers=36, period=8):
    """Full on exactly one seeded step of every aligned run of ``period`` steps (steps
    8k .. 8k+7 at the default period): 128 of 1024 steps, and the 12.5 % rate holds in
    every window that starts at step 0 and spans whole runs."""
    wid = 3
    g = np_rng(wid, C_SCHED)
    runs = -(-steps // period)
    chosen = np.arange(runs) * period + g.integers(0, period, size=runs)
    chosen = chosen[chosen < steps]
    sched = -np.ones(steps, np.float32)
    sched[chosen] = 1.0
    mb = _blocks_for(H0 + steps)
    return Workload(wid, "oda_stack128k", layers=layers, batch=1, Hq=32, Hkv=8, steps=steps, passes=2,
                    H0=np.array([H0], np.int64),
                    block_tables=np.arange(mb, dtype=np.int32)[None, :], num_phys_blocks=mb,
                    sched_scores=sched[:, None])


def da_32k(steps=512, prompt_blocks=1984, output_blocks=64, focus_blocks=128, local_tokens=1024):
    wid = 4
    H0 = (prompt_blocks + output_blocks) * BLOCK
    mb = _blocks_for(H0 + steps)
    perm = np_rng(wid, C_PERM).permutation(mb).astype(np.int32)
    g = np_rng(wid, C_MODE)
    modes = g.integers(0, 3, size=steps)
    f0 = g.integers(0, prompt_blocks - focus_blocks + 1, size=steps)
    decl = np.zeros((steps, 1, 4), np.int32)
    for t in range(steps):
        if modes[t] == DA_FOCUS:
            decl[t, 0] = (DA_FOCUS, f0[t], f0[t] + focus_blocks, prompt_blocks)
        else:
            decl[t, 0] = (modes[t], 0, 0, prompt_blocks)
    return Workload(wid, "da_32k", layers=1, batch=1, Hq=32, Hkv=8, steps=steps, passes=1,
                    H0=np.array([H0], np.int64), block_tables=perm[None, :], num_phys_blocks=mb,
                    decl=decl, da_local_tokens=local_tokens,
                    extra=dict(prompt_blocks=prompt_blocks))


def da_tags_32k(steps=512, prompt_blocks=1984, output_blocks=64, num_segments=16, local_tokens=1024,
                tag_rate=0.06):
    """The ``da_32k`` shape driven by a declaration stream: 16 named segments ("Magic
    Chunks") of 256-4096 positions at seeded, block-unaligned offsets of the prompt;
    per step the input token is a mode tag with probability ``tag_rate`` (global,
    focus, local equally likely), a focus tag is followed by a segment token (a valid
    segment with probability 0.85, else an out-of-range segment id or an ordinary
    token), and ordinary tokens are uniform in [1000, 50000)."""
    wid = 6
    H0 = (prompt_blocks + output_blocks) * BLOCK
    mb = _blocks_for(H0 + steps)
    perm = np_rng(wid, C_PERM).permutation(mb).astype(np.int32)
    g = np_rng(wid, C_SEGMENTS)
    lens = g.integers(256, 4097, size=num_segments)
    begins = g.integers(0, prompt_blocks * BLOCK - 4096, size=num_segments)
    segments = np.stack([begins, begins + lens], axis=1).astype(np.int32)[None]
    g = np_rng(wid, C_TOKENS)
    tokens = np.zeros((steps, 1), np.int32)
    t = 0
    while t < steps:
        if g.random() < tag_rate:
            tag = (TAG_GLOBAL, TAG_FOCUS, TAG_LOCAL)[int(g.integers(0, 3))]
            tokens[t, 0] = tag
            if tag == TAG_FOCUS and t + 1 < steps:
                t += 1
                u = g.random()
                if u < 0.85:
                    tokens[t, 0] = TAG_SEGMENT_BASE + int(g.integers(0, num_segments))
                elif u < 0.95:
                    tokens[t, 0] = TAG_SEGMENT_BASE + num_segments + int(g.integers(0, 4))
                else:
                    tokens[t, 0] = int(g.integers(1000, 50000))
        else:
            tokens[t, 0] = int(g.integers(1000, 50000))
        t += 1
    return Workload(wid, "da_tags_32k", layers=1, batch=1, Hq=32, Hkv=8, steps=steps, passes=1,
                    H0=np.array([H0], np.int64), block_tables=perm[None, :], num_phys_blocks=mb,
                    da_local_tokens=local_tokens, tokens=tokens, segments=segments,
                    output_begin=np.array([prompt_blocks], np.int32),
                    da_tags=(TAG_GLOBAL, TAG_FOCUS, TAG_LOCAL, TAG_SEGMENT_BASE),
                    extra=dict(prompt_blocks=prompt_blocks))


def ragged32(steps=256, batch=32, lo=4096, hi=131072, keep_lo=0.05, keep_hi=0.20):
    wid = 5
    g = np_rng(wid, C_LEN)
    H0 = np.floor(np.exp(g.uniform(math.log(lo), math.log(hi), size=batch))).astype(np.int64)
    nblocks = np.array([_blocks_for(int(h) + steps) for h in H0])
    mb = int(nblocks.max())
    total = int(nblocks.sum())
    perm = np_rng(wid, C_PERM).permutation(total).astype(np.int32)
    bt = np.full((batch, mb), -1, np.int32)
    off = 0
    for r in range(batch):
        bt[r, :nblocks[r]] = perm[off:off + nblocks[r]]
        off += nblocks[r]
    fallback = np.where(np_rng(wid, C_FALLBACK).random(batch) < 0.5, MODE_LOCAL, MODE_BLOCKS).astype(np.int32)
    words = (mb + 31) // 32
    keep = np.zeros((batch, words), np.uint32)
    fracs = np.zeros(batch)
    for r in range(batch):
        gk = np_rng(wid, C_KEEP, r)
        f = gk.uniform(keep_lo, keep_hi)
        existing = _blocks_for(int(H0[r]))
        k = max(1, int(round(f * existing)))
        kept = set(gk.choice(existing, size=k, replace=False).tolist())
        kept |= set(range(int(H0[r]) // BLOCK, mb))
        for blk in kept:
            keep[r, blk // 32] |= np.uint32(1 << (blk % 32))
        fracs[r] = f
    return Workload(wid, "ragged32", layers=1, batch=batch, Hq=32, Hkv=8, steps=steps, passes=1,
                    H0=H0, block_tables=bt, num_phys_blocks=total, fallback=fallback, keep_mask=keep,
                    extra=dict(keep_fraction=fracs))


ALL = {w.__name__: w for w in (oda_small, oda_stack16k, oda_stack128k, da_32k, ragged32)}
