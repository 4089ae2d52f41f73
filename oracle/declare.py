"""Declarative-Attention declarations read from the generated tokens (oracle side).

DA review page, section 1 "Key Terms": generation is split into three declared
modes -- global (the whole context), focus (one named context segment, a "Magic
Chunk"), local (only the model's own output); section 3 and the chatpaper
abstract: the model writes the mode tags <global>, <focus>, <local> into its
chain of thought and the inference engine parses them like tool calls to build
the attention mask.

Readings (the pages give no grammar):

* a mode tag is one token; the mode holds for the tokens after it until the next
  tag, starting in global mode;
* <focus> is followed by one token naming the segment (``segment_base + k`` for
  segment k); the focus starts when that token arrives. If the token after
  <focus> names no segment the focus declaration is dropped; a new tag before
  the segment token replaces the pending focus;
* a segment [begin, end) of context positions covers the blocks
  [begin // 16, ceil(end / 16)), none when end <= begin;
* the step whose input token completes a declaration already uses it (the
  engine parsed the token when it was generated, before this step runs).

The per-step result is the row (mode, focus_begin_block, focus_end_block,
output_begin_block) that ``gather.da_mode_blocks`` turns into kept blocks.
"""

from .gather import FOCUS, GLOBAL, LOCAL


def parse_declarations(tokens, tags, segments, output_begin_block, block_size=16):
    """Per-step declaration rows and parser states for one request.

    tokens: the input token of each step; tags: (global, focus, local,
    segment_base) token ids; segments: list of (begin, end) positions.
    Returns (rows, states): rows[t] = (mode, fb, fe, output_begin_block),
    states[t] = (mode, fb, fe, pending) after step t.
    """
    g_tag, f_tag, l_tag, seg_base = tags
    mode, fb, fe, pending = GLOBAL, 0, 0, False
    rows, states = [], []
    for tok in tokens:
        tok = int(tok)
        if tok == g_tag:
            mode, pending = GLOBAL, False
        elif tok == l_tag:
            mode, pending = LOCAL, False
        elif tok == f_tag:
            pending = True
        elif pending:
            pending = False
            k = tok - seg_base
            if 0 <= k < len(segments):
                begin, end = int(segments[k][0]), int(segments[k][1])
                begin = max(begin, 0)
                mode = FOCUS
                fb = begin // block_size
                fe = -(-end // block_size) if end > begin else fb
        rows.append((mode, fb, fe, output_begin_block))
        states.append((mode, fb, fe, int(pending)))
    return rows, states
