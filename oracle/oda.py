"""One On-Demand-Attention decode step, layer by layer (oracle side).

ODA summary page, "Approach", inference procedure: at every token the Local
pass runs first (s = 4 initial tokens plus the recent window w = 2048); if the
recall score satisfies q_t > theta, the current step is recomputed from the same
prior state with Full attention and that result is selected; the current
position's KV of the selected pass is committed to the preserved full history,
where later recalls can read it. Figure 1's caption: Local runs at every step
and Full is added selectively.

The commit is modelled exactly as the pages order it: the Local pass writes its
candidate (k, v) into position n-1 and attends; a recall pass overwrites
position n-1 with its own candidate and attends over all n positions. The
position therefore ends up holding the selected pass's candidate.

Ragged batches: each request takes full when its score exceeds theta and
otherwise its own fallback view (local, or a DA block keep-list).
"""

from . import attention, keysets

MODE_LOCAL, MODE_FULL, MODE_BLOCKS = 0, 1, 2


def commit(hist_k, hist_v, n, k_new, v_new):
    """Write the current token's bf16 key/value bits into position n-1."""
    hist_k[n - 1] = k_new
    hist_v[n - 1] = v_new


def local_pass(q, k_new, v_new, hist_k, hist_v, n, scale, sinks=4, window=2048):
    commit(hist_k, hist_v, n, k_new, v_new)
    return attention.attend(q, hist_k, hist_v, keysets.local_keys(n, sinks, window), scale)


def full_pass(q, k_new, v_new, hist_k, hist_v, n, scale):
    commit(hist_k, hist_v, n, k_new, v_new)
    return attention.attend(q, hist_k, hist_v, keysets.full_keys(n), scale)


def recall_pass(q, k_new, v_new, hist_k, hist_v, n, scale, local_only, sinks=4, window=2048):
    """One layer's part of the recall pass under per-layer access control.

    ODA summary page, "Developer perspective", the note on hybrid backbones: the
    runtime may restrict chosen layers to the Local range. Reading: a layer so
    restricted attends its Local view in the recall pass too (it never reads past
    the sinks and the window); the other layers attend the full history. Either way
    the recall pass's candidate is committed.
    """
    if local_only:
        return local_pass(q, k_new, v_new, hist_k, hist_v, n, scale, sinks, window)
    return full_pass(q, k_new, v_new, hist_k, hist_v, n, scale)


def blocks_pass(q, k_new, v_new, hist_k, hist_v, n, kept_blocks, scale, block_size=16):
    """DA step: commit, then attend the kept blocks only."""
    commit(hist_k, hist_v, n, k_new, v_new)
    return attention.attend(q, hist_k, hist_v, keysets.block_keys(n, kept_blocks, block_size), scale)


def select(gate, o_local, o_full):
    """Step output: the Full result when the step recalled, else the Local one."""
    return o_full if gate else o_local


def request_mode(score, theta, fallback):
    """Per-request view for a ragged batch: full when score > theta, else the
    request's fallback view."""
    return MODE_FULL if score > theta else fallback
