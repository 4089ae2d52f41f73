"""Which key positions a decode step attends (oracle side).

Positions are 0-based; ``n`` is the number of keys visible at the step and
includes the current token, whose KV is written to position n-1 before the
step attends (ODA summary page, "Approach": the selected pass's current
position KV is committed to the preserved history; "Main results": the local
window w = 2048 counts the current token).
"""

import numpy as np


def full_keys(n):
    """Full view: every preserved position 0..n-1 (ODA summary page, "Approach",
    the Full recomputation over the whole history)."""
    return np.arange(n, dtype=np.int64)


def local_keys(n, sinks=4, window=2048):
    """Local view: the first ``sinks`` positions plus the last ``window``
    positions, each position once (ODA summary page, "Approach": initial s = 4
    and recent window w = 2048; "Main results": the window includes the current
    token)."""
    first = np.arange(min(sinks, n), dtype=np.int64)
    recent = np.arange(max(0, n - window), n, dtype=np.int64)
    return np.union1d(first, recent)


def block_keys(n, kept_blocks, block_size=16):
    """Block view: all valid positions of the kept KV blocks. Block b holds
    positions 16b .. 16b+15, cut at n (DA review page, section 3: the mask is
    applied per KV block and only kept blocks reach the attention kernel)."""
    out = []
    for b in sorted(set(int(x) for x in kept_blocks)):
        lo, hi = block_size * b, min(block_size * b + block_size, n)
        if lo < hi:
            out.append(np.arange(lo, hi, dtype=np.int64))
    if not out:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(out)
