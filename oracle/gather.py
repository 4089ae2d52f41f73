"""Declarative-Attention keep-sets and the rewritten block list (oracle side).

DA review page, section 3 (and the chatpaper abstract): generation is split
into three declared modes -- global (the whole context), focus (one named
region), local (only the model's recent output) -- and the engine applies the
mask at KV-block granularity by rewriting the block table so that only kept
blocks reach the attention kernel.

Keep-set readings for the synthetic workloads (the pages give no block
arithmetic):

* global: every block that holds at least one visible position;
* focus:  the blocks of one contiguous region [focus_begin, focus_end) plus
          every block of the model's own output, i.e. blocks >= output_begin;
* local:  the blocks that overlap the last ``local_tokens`` positions.
"""

import numpy as np

GLOBAL, FOCUS, LOCAL = 0, 1, 2


def num_blocks(n, block_size=16):
    return (n + block_size - 1) // block_size


def da_mode_blocks(mode, n, focus_begin=0, focus_end=0, output_begin=0,
                   local_tokens=1024, block_size=16):
    """Sorted list of kept logical block ids for one declared mode."""
    nb = num_blocks(n, block_size)
    if mode == GLOBAL:
        kept = set(range(nb))
    elif mode == FOCUS:
        kept = set(range(max(0, focus_begin), min(focus_end, nb)))
        kept |= set(range(max(0, output_begin), nb))
    elif mode == LOCAL:
        first = max(0, n - local_tokens) // block_size
        kept = set(range(first, nb))
    else:
        raise ValueError("unknown mode %r" % (mode,))
    return sorted(kept)


def mask_to_blocks(mask_words, n, block_size=16):
    """Kept block ids from a little-endian bit mask (bit b of word b//32),
    restricted to blocks that hold visible positions."""
    nb = num_blocks(n, block_size)
    out = []
    for b in range(nb):
        if (int(mask_words[b // 32]) >> (b % 32)) & 1:
            out.append(b)
    return out


def gather_blocks(block_table, kept, n, block_size=16):
    """The rewritten block list: for each kept logical block b in ascending
    order, (physical id block_table[b], number of valid positions in b)."""
    phys, cnt = [], []
    for b in sorted(set(int(x) for x in kept)):
        lo = block_size * b
        if lo >= n:
            continue
        phys.append(int(block_table[b]))
        cnt.append(min(block_size, n - lo))
    return np.asarray(phys, dtype=np.int32), np.asarray(cnt, dtype=np.int32)
