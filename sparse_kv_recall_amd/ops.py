"""Torch-facing binding of libsparsekv: same names as the C ABI, argument marshalling only.

Tensors must live on the GPU; every step of the computation runs in the HIP
library on torch's current stream. Nothing here computes a result.
"""

import math

import torch

from . import _lib

BLOCK = 16
HEAD_DIM = 128
TILE_ELEMS = BLOCK * HEAD_DIM

MODE_LOCAL, MODE_FULL, MODE_BLOCKS = 0, 1, 2
DA_GLOBAL, DA_FOCUS, DA_LOCAL = 0, 1, 2


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def _check(t, dtype, name, numel=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if numel is not None and t.numel() < numel:
        raise ValueError("%s has %d elements, needs %d" % (name, t.numel(), numel))


class PagedKVCache:
    """Device memory of one paged bf16 KV cache (one attention layer).

    k_pool / v_pool: bf16 [num_phys_blocks][num_kv_heads][16*128] tiles in the
    library's tile order; block_tables: int32 [batch][max_blocks];
    seq_lens: int32 [batch] (visible positions, current token included).
    """

    def __init__(self, num_phys_blocks, batch, num_q_heads, num_kv_heads, max_blocks, device="cuda",
                 block_tables=None, seq_lens=None, k_pool=None, v_pool=None):
        self.num_phys_blocks = int(num_phys_blocks)
        self.batch = int(batch)
        self.num_q_heads = int(num_q_heads)
        self.num_kv_heads = int(num_kv_heads)
        self.max_blocks = int(max_blocks)
        shape = (self.num_phys_blocks, self.num_kv_heads, TILE_ELEMS)
        self.k_pool = k_pool if k_pool is not None else torch.empty(shape, dtype=torch.bfloat16, device=device)
        self.v_pool = v_pool if v_pool is not None else torch.empty(shape, dtype=torch.bfloat16, device=device)
        self.block_tables = (block_tables if block_tables is not None else
                             torch.zeros((self.batch, self.max_blocks), dtype=torch.int32, device=device))
        self.seq_lens = (seq_lens if seq_lens is not None else
                         torch.zeros(self.batch, dtype=torch.int32, device=device))
        _check(self.k_pool, torch.bfloat16, "k_pool", self.num_phys_blocks * self.num_kv_heads * TILE_ELEMS)
        _check(self.v_pool, torch.bfloat16, "v_pool", self.num_phys_blocks * self.num_kv_heads * TILE_ELEMS)
        _check(self.block_tables, torch.int32, "block_tables", self.batch * self.max_blocks)
        _check(self.seq_lens, torch.int32, "seq_lens", self.batch)

    def abi(self):
        return _lib.PagedKVStruct(self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.block_tables.data_ptr(),
                                  self.seq_lens.data_ptr(), self.batch, self.num_q_heads, self.num_kv_heads,
                                  HEAD_DIM, BLOCK, self.max_blocks, self.num_phys_blocks)

    def nbytes(self):
        return self.k_pool.numel() * 2 * 2


def workspace_bytes(batch, num_q_heads):
    return int(_lib.load().sk_workspace_bytes(int(batch), int(num_q_heads)))


def workspace(batch, num_q_heads, device="cuda"):
    """Allocate and clear a workspace for calls on up to `batch` requests."""
    n = workspace_bytes(batch, num_q_heads)
    ws = torch.empty(n, dtype=torch.uint8, device=device)
    _lib.call("sk_workspace_init", ws.data_ptr(), n, _stream(ws.device))
    return ws


def workspace_error(ws):
    """SK_DEVERR_* bits of the workspace (synchronizes the current stream)."""
    import ctypes
    v = ctypes.c_int32(0)
    _lib.call("sk_workspace_error", ws.data_ptr(), ctypes.addressof(v), _stream(ws.device))
    return int(v.value)


def kv_write(kv, request, pos0, k, v, ws=None):
    count = k.shape[0]
    _check(k, torch.bfloat16, "k", count * kv.num_kv_heads * HEAD_DIM)
    _check(v, torch.bfloat16, "v", count * kv.num_kv_heads * HEAD_DIM)
    _lib.call("sk_kv_write", kv.abi(), int(request), int(pos0), int(count), k.data_ptr(), v.data_ptr(), _ptr(ws),
              _stream(k.device))


def kv_read(kv, request, pos0, count, ws=None):
    k = torch.empty((count, kv.num_kv_heads, HEAD_DIM), dtype=torch.bfloat16, device=kv.k_pool.device)
    v = torch.empty_like(k)
    _lib.call("sk_kv_read", kv.abi(), int(request), int(pos0), int(count), k.data_ptr(), v.data_ptr(), _ptr(ws),
              _stream(k.device))
    return k, v


def kv_append(kv, k_new, v_new, sel=None, sel_value=1, ws=None):
    n = kv.batch * kv.num_kv_heads * HEAD_DIM
    _check(k_new, torch.bfloat16, "k_new", n)
    _check(v_new, torch.bfloat16, "v_new", n)
    _check(sel, torch.int32, "sel", kv.batch)
    _lib.call("sk_kv_append", kv.abi(), k_new.data_ptr(), v_new.data_ptr(), _ptr(sel), int(sel_value), _ptr(ws),
              _stream(k_new.device))


def _decode_common(q, kv, k_new, v_new, sel, out, ws):
    _check(q, torch.float32, "q", kv.batch * kv.num_q_heads * HEAD_DIM)
    n = kv.batch * kv.num_kv_heads * HEAD_DIM
    _check(k_new, torch.bfloat16, "k_new", n)
    _check(v_new, torch.bfloat16, "v_new", n)
    _check(sel, torch.int32, "sel", kv.batch)
    if out is None:
        out = torch.zeros((kv.batch, kv.num_q_heads, HEAD_DIM), dtype=torch.float32, device=q.device)
    _check(out, torch.float32, "out", kv.batch * kv.num_q_heads * HEAD_DIM)
    if ws is None:
        ws = workspace(kv.batch, kv.num_q_heads, q.device)
    _check(ws, torch.uint8, "ws")
    return out, ws


def oda_decode_local(q, kv, k_new=None, v_new=None, sinks=4, window=2048, scale=None, sel=None,
                     sel_value=MODE_LOCAL, out=None, ws=None):
    out, ws = _decode_common(q, kv, k_new, v_new, sel, out, ws)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_local", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), int(sinks), int(window), scale,
              _ptr(sel), int(sel_value), out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device))
    return out


def local_tiles_bytes(batch, sinks, window, max_blocks):
    return int(_lib.load().oda_local_tiles_bytes(int(batch), int(sinks), int(window), int(max_blocks)))


def local_tiles(kv, sinks=4, window=2048, tab=None):
    """The Local view's tile table of the current step (oda_local_tiles): one int32 row per
    request, shared by every layer with the same block tables and lengths."""
    n = local_tiles_bytes(kv.batch, sinks, window, kv.max_blocks)
    if n == 0:
        raise ValueError("invalid sinks / window / shape for a Local tile table")
    if tab is None:
        tab = torch.zeros(n // 4, dtype=torch.int32, device=kv.block_tables.device)
    _check(tab, torch.int32, "tab")
    if tab.numel() * 4 < n:
        raise ValueError("tile table too small: %d bytes needed" % n)
    _lib.call("oda_local_tiles", kv.abi(), int(sinks), int(window), tab.data_ptr(), tab.numel() * 4,
              _stream(tab.device))
    return tab


def oda_decode_local_tiles(q, kv, tab, k_new=None, v_new=None, sinks=4, window=2048, scale=None, sel=None,
                           sel_value=MODE_LOCAL, out=None, ws=None):
    """oda_decode_local with the step's tile table (local_tiles): the same results."""
    if tab is None:
        raise ValueError("tab is required (ops.local_tiles)")
    out, ws = _decode_common(q, kv, k_new, v_new, sel, out, ws)
    _check(tab, torch.int32, "tab")
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_local_tiles", q.data_ptr(), kv.abi(), tab.data_ptr(), tab.numel() * 4, _ptr(k_new),
              _ptr(v_new), int(sinks), int(window), scale, _ptr(sel), int(sel_value), out.data_ptr(),
              ws.data_ptr(), ws.numel(), _stream(q.device))
    return out


def oda_decode_full(q, kv, k_new=None, v_new=None, scale=None, sel=None, sel_value=1, out=None, ws=None):
    out, ws = _decode_common(q, kv, k_new, v_new, sel, out, ws)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_full", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), scale, _ptr(sel),
              int(sel_value), out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device))
    return out


def _qkv_common(qkv, g_q, g_k, kv, sel, out, ws):
    heads = kv.num_q_heads + 2 * kv.num_kv_heads
    _check(qkv, torch.float32, "qkv", kv.batch * heads * HEAD_DIM)
    _check(g_q, torch.bfloat16, "g_q", HEAD_DIM)
    _check(g_k, torch.bfloat16, "g_k", HEAD_DIM)
    if qkv is None or g_q is None or g_k is None:
        raise ValueError("qkv, g_q and g_k are required")
    return _decode_common(qkv, kv, None, None, sel, out, ws)


def oda_decode_local_qkv(qkv, g_q, g_k, kv, eps=1e-6, rope_base=1.0e6, sinks=4, window=2048, scale=None, sel=None,
                         sel_value=MODE_LOCAL, out=None, ws=None):
    """oda_decode_local from a layer's raw q/k/v projection qkv [B][Hq + 2 Hkv][128] fp32:
    per-head RMSNorm (gains g_q, g_k) and rotary positions at n - 1 are applied on load,
    and the finished k and v (bf16) are committed at n - 1."""
    out, ws = _qkv_common(qkv, g_q, g_k, kv, sel, out, ws)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_local_qkv", qkv.data_ptr(), g_q.data_ptr(), g_k.data_ptr(), float(eps), float(rope_base),
              kv.abi(), int(sinks), int(window), scale, _ptr(sel), int(sel_value), out.data_ptr(), ws.data_ptr(),
              ws.numel(), _stream(qkv.device))
    return out


def oda_decode_full_qkv(qkv, g_q, g_k, kv, eps=1e-6, rope_base=1.0e6, scale=None, sel=None, sel_value=1, out=None,
                        ws=None):
    """oda_decode_full from a layer's raw q/k/v projection (see oda_decode_local_qkv)."""
    out, ws = _qkv_common(qkv, g_q, g_k, kv, sel, out, ws)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_full_qkv", qkv.data_ptr(), g_q.data_ptr(), g_k.data_ptr(), float(eps), float(rope_base),
              kv.abi(), scale, _ptr(sel), int(sel_value), out.data_ptr(), ws.data_ptr(), ws.numel(),
              _stream(qkv.device))
    return out


def oda_decode_full_noalloc(q, kv, out, k_new=None, v_new=None, scale=None, sel=None, sel_value=1, dev_err=None):
    """oda_decode_full without a workspace (the library's own device array serves as one);
    `out` is required, so nothing is allocated on this path."""
    _check(q, torch.float32, "q", kv.batch * kv.num_q_heads * HEAD_DIM)
    n = kv.batch * kv.num_kv_heads * HEAD_DIM
    _check(k_new, torch.bfloat16, "k_new", n)
    _check(v_new, torch.bfloat16, "v_new", n)
    _check(sel, torch.int32, "sel", kv.batch)
    _check(out, torch.float32, "out", kv.batch * kv.num_q_heads * HEAD_DIM)
    _check(dev_err, torch.int32, "dev_err", 1)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_full_noalloc", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), scale, _ptr(sel),
              int(sel_value), out.data_ptr(), _ptr(dev_err), _stream(q.device))
    return out


def oda_recall_score(x, W1, b1, w2, b2, theta=0.0, q_out=None, gate_out=None, ws=None):
    batch, in_dim = x.shape
    hidden = W1.shape[0]
    for t, name, n in ((x, "x", batch * in_dim), (W1, "W1", hidden * in_dim), (b1, "b1", hidden),
                       (w2, "w2", hidden), (b2, "b2", 1)):
        _check(t, torch.float32, name, n)
    if q_out is None:
        q_out = torch.empty(batch, dtype=torch.float32, device=x.device)
    if gate_out is None:
        gate_out = torch.empty(batch, dtype=torch.int32, device=x.device)
    _check(q_out, torch.float32, "q_out", batch)
    _check(gate_out, torch.int32, "gate_out", batch)
    if ws is None:
        ws = workspace(batch, 1, x.device)
    _lib.call("oda_recall_score", x.data_ptr(), W1.data_ptr(), b1.data_ptr(), w2.data_ptr(), b2.data_ptr(),
              int(batch), int(in_dim), int(hidden), float(theta), q_out.data_ptr(), gate_out.data_ptr(),
              ws.data_ptr(), ws.numel(), _stream(x.device))
    return q_out, gate_out


def oda_gate_scores(scores, theta=0.0, fallback=None, out=None):
    batch = scores.numel()
    _check(scores, torch.float32, "scores", batch)
    _check(fallback, torch.int32, "fallback", batch)
    if out is None:
        out = torch.empty(batch, dtype=torch.int32, device=scores.device)
    _check(out, torch.int32, "out", batch)
    _lib.call("oda_gate_scores", scores.data_ptr(), int(batch), float(theta), _ptr(fallback), out.data_ptr(),
              _stream(scores.device))
    return out


def da_keep_mask(decl, kv, local_tokens=1024, mask=None):
    words = (kv.max_blocks + 31) // 32
    _check(decl, torch.int32, "decl", kv.batch * 4)
    if mask is None:
        mask = torch.empty((kv.batch, words), dtype=torch.int32, device=decl.device)
    _check(mask, torch.int32, "mask", kv.batch * words)
    _lib.call("da_keep_mask", decl.data_ptr(), kv.abi(), int(local_tokens), mask.data_ptr(), _stream(decl.device))
    return mask


def da_declare(tokens, state, output_begin, kv, tags, segments=None, local_tokens=1024, decl=None, mask=None,
               with_mask=True):
    """Advance each request's declaration parser by this step's token and write the
    step's declaration and (with_mask) keep mask. tokens: int32 [B]; state: int32 [B][4]
    (persistent, start {DA_GLOBAL, 0, 0, 0}); output_begin: int32 [B]; tags:
    (global, focus, local, segment_base) token ids; segments: int32 [B][S][2] or None.
    Returns (decl, mask), mask None without with_mask."""
    B = kv.batch
    words = (kv.max_blocks + 31) // 32
    _check(tokens, torch.int32, "tokens", B)
    _check(state, torch.int32, "state", B * 4)
    _check(output_begin, torch.int32, "output_begin", B)
    nseg = 0
    if segments is not None:
        if segments.dim() != 3 or segments.shape[0] != B or segments.shape[2] != 2:
            raise ValueError("segments must be int32 [batch][num_segments][2]")
        _check(segments, torch.int32, "segments", segments.numel())
        nseg = int(segments.shape[1])
    if decl is None:
        decl = torch.empty((B, 4), dtype=torch.int32, device=tokens.device)
    _check(decl, torch.int32, "decl", B * 4)
    if not with_mask:
        mask = None
    elif mask is None:
        mask = torch.empty((B, words), dtype=torch.int32, device=tokens.device)
    _check(mask, torch.int32, "mask", B * words)
    t = _lib.DaTagsStruct(*(int(x) for x in tags))
    _lib.call("da_declare", tokens.data_ptr(), state.data_ptr(), 0 if segments is None else segments.data_ptr(),
              nseg, output_begin.data_ptr(), t, kv.abi(), int(local_tokens), decl.data_ptr(), _ptr(mask),
              _stream(tokens.device))
    return decl, mask


def da_decode_blocks(q, kv, keep_mask, k_new=None, v_new=None, scale=None, sel=None, sel_value=MODE_BLOCKS,
                     out=None, gathered=None, gathered_cnt=None, num_kept=None, ws=None):
    out, ws = _decode_common(q, kv, k_new, v_new, sel, out, ws)
    words = (kv.max_blocks + 31) // 32
    _check(keep_mask, torch.int32, "keep_mask", kv.batch * words)
    dev = q.device
    if gathered is None:
        gathered = torch.zeros((kv.batch, kv.max_blocks), dtype=torch.int32, device=dev)
    if gathered_cnt is None:
        gathered_cnt = torch.zeros((kv.batch, kv.max_blocks), dtype=torch.int32, device=dev)
    if num_kept is None:
        num_kept = torch.zeros(kv.batch, dtype=torch.int32, device=dev)
    _check(gathered, torch.int32, "gathered", kv.batch * kv.max_blocks)
    _check(gathered_cnt, torch.int32, "gathered_cnt", kv.batch * kv.max_blocks)
    _check(num_kept, torch.int32, "num_kept", kv.batch)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("da_decode_blocks", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), keep_mask.data_ptr(),
              gathered.data_ptr(), gathered_cnt.data_ptr(), num_kept.data_ptr(), scale, _ptr(sel), int(sel_value),
              out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(dev))
    return out, gathered, gathered_cnt, num_kept


def da_gather(kv, keep_mask, gathered=None, gathered_cnt=None, num_kept=None, sel=None, sel_value=MODE_BLOCKS,
              ws=None):
    """The block-table rewrite of da_decode_blocks alone (once per step for all layers)."""
    words = (kv.max_blocks + 31) // 32
    _check(keep_mask, torch.int32, "keep_mask", kv.batch * words)
    dev = keep_mask.device
    if gathered is None:
        gathered = torch.zeros((kv.batch, kv.max_blocks), dtype=torch.int32, device=dev)
    if gathered_cnt is None:
        gathered_cnt = torch.zeros((kv.batch, kv.max_blocks), dtype=torch.int32, device=dev)
    if num_kept is None:
        num_kept = torch.zeros(kv.batch, dtype=torch.int32, device=dev)
    _check(gathered, torch.int32, "gathered", kv.batch * kv.max_blocks)
    _check(gathered_cnt, torch.int32, "gathered_cnt", kv.batch * kv.max_blocks)
    _check(num_kept, torch.int32, "num_kept", kv.batch)
    _check(sel, torch.int32, "sel", kv.batch)
    _lib.call("da_gather", kv.abi(), keep_mask.data_ptr(), gathered.data_ptr(), gathered_cnt.data_ptr(),
              num_kept.data_ptr(), _ptr(sel), int(sel_value), _ptr(ws), _stream(dev))
    return gathered, gathered_cnt, num_kept


def da_decode_gathered(q, kv, gathered, gathered_cnt, num_kept, k_new=None, v_new=None, scale=None, sel=None,
                       sel_value=MODE_BLOCKS, out=None, ws=None):
    """Attention over a gathered block list (da_gather's output), one launch."""
    out, ws = _decode_common(q, kv, k_new, v_new, sel, out, ws)
    _check(gathered, torch.int32, "gathered", kv.batch * kv.max_blocks)
    _check(gathered_cnt, torch.int32, "gathered_cnt", kv.batch * kv.max_blocks)
    _check(num_kept, torch.int32, "num_kept", kv.batch)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("da_decode_gathered", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), gathered.data_ptr(),
              gathered_cnt.data_ptr(), num_kept.data_ptr(), scale, _ptr(sel), int(sel_value), out.data_ptr(),
              ws.data_ptr(), ws.numel(), _stream(q.device))
    return out


def oda_decode_views(q, kv, view, gathered, gathered_cnt, num_kept, k_new=None, v_new=None, sinks=4, window=2048,
                     scale=None, out=None, ws=None):
    """Per-request views in one launch: request b attends Full, Local or its gathered
    block list as view[b] is MODE_FULL, MODE_LOCAL or MODE_BLOCKS (any other value: b
    does not run); the lists are da_gather's output for the MODE_BLOCKS requests."""
    _check(view, torch.int32, "view", kv.batch)
    out, ws = _decode_common(q, kv, k_new, v_new, view, out, ws)
    _check(gathered, torch.int32, "gathered", kv.batch * kv.max_blocks)
    _check(gathered_cnt, torch.int32, "gathered_cnt", kv.batch * kv.max_blocks)
    _check(num_kept, torch.int32, "num_kept", kv.batch)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("oda_decode_views", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), int(sinks), int(window), scale,
              view.data_ptr(), gathered.data_ptr(), gathered_cnt.data_ptr(), num_kept.data_ptr(), out.data_ptr(),
              ws.data_ptr(), ws.numel(), _stream(q.device))
    return out


def da_decode_declared(q, kv, decl, local_tokens=1024, k_new=None, v_new=None, scale=None, sel=None,
                       sel_value=MODE_BLOCKS, out=None, ws=None):
    """Attention over the blocks a declared mode keeps (decl int32 [B][4] as for
    da_keep_mask), the block-table rewrite done in the kernel: one launch."""
    out, ws = _decode_common(q, kv, k_new, v_new, sel, out, ws)
    _check(decl, torch.int32, "decl", 4 * kv.batch)
    scale = 1.0 / math.sqrt(HEAD_DIM) if scale is None else float(scale)
    _lib.call("da_decode_declared", q.data_ptr(), kv.abi(), _ptr(k_new), _ptr(v_new), decl.data_ptr(),
              int(local_tokens), scale, _ptr(sel), int(sel_value), out.data_ptr(), ws.data_ptr(), ws.numel(),
              _stream(q.device))
    return out


# ---- dense layers of the weight-bearing decode step (batch 1)

PRO_NONE, PRO_RMSNORM = 0, 1
EPI_STORE, EPI_SWIGLU = 0, 1


def _sel_args(sel, sel_value):
    if sel is not None:
        _check(sel, torch.int32, "sel", 1)
    return (0 if sel is None else sel.data_ptr()), int(sel_value)


def gemv(W, x, y, prologue=PRO_NONE, gamma=None, eps=1e-6, residual=None, epilogue=EPI_STORE, sel=None,
         sel_value=1):
    """y[r] = W[r] . x' (+ residual[r]) with x' = x or RMSNorm(x) * gamma; with
    EPI_SWIGLU, W holds 2*rows rows and y[r] = SiLU(W[r] . x') * (W[rows + r] . x')."""
    wr, cols = W.shape
    rows = wr // 2 if epilogue == EPI_SWIGLU else wr
    _check(W, torch.bfloat16, "W")
    _check(x, torch.float32, "x", cols)
    _check(y, torch.float32, "y", rows)
    _check(gamma, torch.bfloat16, "gamma", cols)
    _check(residual, torch.float32, "residual", rows)
    s, sv = _sel_args(sel, sel_value)
    _lib.call("sk_gemv", W.data_ptr(), rows, cols, x.data_ptr(), int(prologue), _ptr(gamma), float(eps),
              _ptr(residual), int(epilogue), y.data_ptr(), s, sv, _stream(W.device))
    return y


def qkv_rope(W_qkv, h, g_attn, g_q, g_k, q_heads, kv_heads, seq_lens, scratch, q_out, k_out, v_out, eps=1e-6,
             rope_base=1.0e6, sel=None, sel_value=1):
    """Attention inputs of one token (RMSNorm, q/k/v projection into scratch, per-head q/k
    norm, RoPE at position seq_lens[0] - 1); q_out fp32 [Hq*128], k_out / v_out bf16
    [Hkv*128]; scratch fp32 [(Hq + 2 Hkv) * 128]."""
    hidden = h.numel()
    heads = q_heads + 2 * kv_heads
    _check(W_qkv, torch.bfloat16, "W_qkv", heads * HEAD_DIM * hidden)
    _check(h, torch.float32, "h")
    for t, n in ((g_attn, hidden), (g_q, HEAD_DIM), (g_k, HEAD_DIM)):
        _check(t, torch.bfloat16, "gamma", n)
    _check(seq_lens, torch.int32, "seq_lens", 1)
    _check(scratch, torch.float32, "scratch", heads * HEAD_DIM)
    _check(q_out, torch.float32, "q_out", q_heads * HEAD_DIM)
    _check(k_out, torch.bfloat16, "k_out", kv_heads * HEAD_DIM)
    _check(v_out, torch.bfloat16, "v_out", kv_heads * HEAD_DIM)
    s, sv = _sel_args(sel, sel_value)
    _lib.call("sk_qkv_rope", W_qkv.data_ptr(), h.data_ptr(), g_attn.data_ptr(), g_q.data_ptr(), g_k.data_ptr(),
              hidden, int(q_heads), int(kv_heads), float(eps), float(rope_base), seq_lens.data_ptr(),
              scratch.data_ptr(), q_out.data_ptr(), k_out.data_ptr(), v_out.data_ptr(), s, sv, _stream(h.device))


def rmsnorm(x, gamma, out, eps=1e-6, sel=None, sel_value=1):
    _check(x, torch.float32, "x")
    _check(gamma, torch.bfloat16, "gamma", x.numel())
    _check(out, torch.float32, "out", x.numel())
    s, sv = _sel_args(sel, sel_value)
    _lib.call("sk_rmsnorm", x.data_ptr(), gamma.data_ptr(), x.numel(), float(eps), out.data_ptr(), s, sv,
              _stream(x.device))
    return out


def embed(table, token, out, out2=None, sel=None, sel_value=1):
    vocab, hidden = table.shape
    _check(table, torch.bfloat16, "table")
    _check(token, torch.int32, "token", 1)
    _check(out, torch.float32, "out", hidden)
    _check(out2, torch.float32, "out2", hidden)
    s, sv = _sel_args(sel, sel_value)
    _lib.call("sk_embed", table.data_ptr(), vocab, hidden, token.data_ptr(), out.data_ptr(), _ptr(out2), s, sv,
              _stream(out.device))
    return out


STREAM_READ_GRID = 256  # workgroups (and checksum words) of sk_stream_read


def stream_read(data, sink=None):
    """Bandwidth reference: reads every byte of the contiguous device tensor `data` once;
    returns the int32 [STREAM_READ_GRID] per-workgroup XOR checksums (sk_stream_read)."""
    if not data.is_contiguous():
        raise ValueError("data must be contiguous")
    if sink is None:
        sink = torch.empty(STREAM_READ_GRID, dtype=torch.int32, device=data.device)
    _check(sink, torch.int32, "sink", STREAM_READ_GRID)
    nbytes = data.numel() * data.element_size()
    _lib.call("sk_stream_read", data.data_ptr(), nbytes, sink.data_ptr(), _stream(data.device))
    return sink


def select(gate, a, b, out, gate_value=1):
    _check(gate, torch.int32, "gate", 1)
    for t, n in ((a, "a"), (b, "b"), (out, "out")):
        _check(t, torch.float32, n, out.numel())
    _lib.call("sk_select", gate.data_ptr(), int(gate_value), a.data_ptr(), b.data_ptr(), out.numel(),
              out.data_ptr(), _stream(out.device))
    return out
