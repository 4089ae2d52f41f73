"""CPU checks of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments with the documented codes before touching a GPU."""

import ctypes

import pytest

from sparse_kv_recall_amd import _lib

SK_E_NULL, SK_E_SHAPE, SK_E_HEADS, SK_E_RANGE, SK_E_WORKSPACE = -1, -2, -3, -4, -5
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def lib():
    try:
        return _lib.load()
    except _lib.LibraryMissing as e:
        pytest.fail(str(e))


def test_exports_every_header_function():
    names = _lib.header_functions()
    assert len(names) >= 13
    L = lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(_lib._SIGNATURES) == set(names)


def kv(**over):
    d = dict(k_pool=FAKE, v_pool=FAKE, block_tables=FAKE, seq_lens=FAKE, batch=1, num_q_heads=32,
             num_kv_heads=8, head_dim=128, block_size=16, max_blocks=100, num_phys_blocks=100)
    d.update(over)
    return _lib.PagedKVStruct(**d)


def decode_full(k, ws_bytes=1 << 30, q=FAKE, out=FAKE, ws=FAKE):
    return lib().oda_decode_full(q, k, None, None, 0.1, None, 1, out, ws, ws_bytes, None)


def test_decode_argument_validation():
    assert decode_full(kv(k_pool=None)) == SK_E_NULL
    assert decode_full(kv(), q=None) == SK_E_NULL
    assert decode_full(kv(head_dim=64)) == SK_E_SHAPE
    assert decode_full(kv(block_size=32)) == SK_E_SHAPE
    assert decode_full(kv(num_q_heads=12)) == SK_E_HEADS
    assert decode_full(kv(num_q_heads=64, num_kv_heads=2)) == SK_E_SHAPE  # group 32 > 16
    assert decode_full(kv(batch=0)) == SK_E_RANGE
    assert decode_full(kv(max_blocks=0)) == SK_E_RANGE
    assert decode_full(kv(), ws_bytes=16) == SK_E_WORKSPACE
    L = lib()
    assert L.oda_decode_local(FAKE, kv(), None, None, -1, 2048, 0.1, None, 0, FAKE, FAKE, 1 << 30, None) == SK_E_RANGE
    assert L.oda_decode_local(FAKE, kv(), None, None, 4, 0, 0.1, None, 0, FAKE, FAKE, 1 << 30, None) == SK_E_RANGE
    # k_new without v_new
    assert L.oda_decode_local(FAKE, kv(), FAKE, None, 4, 2048, 0.1, None, 0, FAKE, FAKE, 1 << 30, None) == SK_E_NULL
    # per-request views: the view array and the gathered lists are required
    views = lambda view=FAKE, gat=FAKE, sinks=4, window=2048, k=kv(): L.oda_decode_views(
        FAKE, k, None, None, sinks, window, 0.1, view, gat, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert views(view=None) == SK_E_NULL
    assert views(gat=None) == SK_E_NULL
    assert views(sinks=-1) == SK_E_RANGE
    assert views(window=0) == SK_E_RANGE
    assert views(k=kv(num_q_heads=12)) == SK_E_HEADS


def test_local_tiles_validation_and_size():
    # the Local view's tile table: one row of 3 + (sink blocks + window blocks + 1) words per
    # request, capped at max_blocks tiles; its builder and the decode that reads it check
    # their arguments before any HIP call
    L = lib()
    assert L.oda_local_tiles_bytes(1, 4, 2048, 8194) == (3 + 1 + 128 + 1) * 4
    assert L.oda_local_tiles_bytes(3, 0, 20, 8194) == 3 * (3 + 0 + 2 + 1) * 4
    assert L.oda_local_tiles_bytes(1, 4, 2048, 10) == (3 + 10) * 4
    assert L.oda_local_tiles_bytes(0, 4, 2048, 100) == 0 and L.oda_local_tiles_bytes(1, -1, 2048, 100) == 0
    assert L.oda_local_tiles_bytes(1, 4, 0, 100) == 0
    need = L.oda_local_tiles_bytes(1, 4, 2048, 100)
    assert L.oda_local_tiles(kv(), 4, 2048, None, need, None) == SK_E_NULL
    assert L.oda_local_tiles(kv(k_pool=None), 4, 2048, FAKE, need, None) == SK_E_NULL
    assert L.oda_local_tiles(kv(), -1, 2048, FAKE, need, None) == SK_E_RANGE
    assert L.oda_local_tiles(kv(), 4, 0, FAKE, need, None) == SK_E_RANGE
    assert L.oda_local_tiles(kv(), 4, 2048, FAKE, need - 4, None) == SK_E_WORKSPACE
    dec = lambda tab=FAKE, tab_bytes=need, sinks=4, window=2048, k=kv(), q=FAKE: L.oda_decode_local_tiles(
        q, k, tab, tab_bytes, None, None, sinks, window, 0.1, None, 0, FAKE, FAKE, 1 << 30, None)
    assert dec(tab=None) == SK_E_NULL
    assert dec(q=None) == SK_E_NULL
    assert dec(sinks=-1) == SK_E_RANGE
    assert dec(window=0) == SK_E_RANGE
    assert dec(tab_bytes=need - 4) == SK_E_WORKSPACE
    assert dec(k=kv(head_dim=64)) == SK_E_SHAPE


def test_decode_full_noalloc_validation():
    # the allocation-free Full view checks its arguments, and the size its device array
    # holds (16 MiB: batch * num_q_heads up to about 15700), before any HIP call
    L = lib()
    call = lambda k, q=FAKE, out=FAKE, kn=None, vn=None: L.oda_decode_full_noalloc(
        q, k, kn, vn, 0.1, None, 1, out, None, None)
    assert call(kv(k_pool=None)) == SK_E_NULL
    assert call(kv(), q=None) == SK_E_NULL
    assert call(kv(), out=None) == SK_E_NULL
    assert call(kv(), kn=FAKE) == SK_E_NULL
    assert call(kv(head_dim=64)) == SK_E_SHAPE
    assert call(kv(num_q_heads=12)) == SK_E_HEADS
    assert call(kv(batch=1024, num_q_heads=32)) == SK_E_WORKSPACE
    assert call(kv(batch=512, num_q_heads=32)) == SK_E_WORKSPACE
    assert L.sk_workspace_bytes(480, 32) <= 16 << 20 < L.sk_workspace_bytes(512, 32)


def test_decode_from_projection_validation():
    # the Local / Full views from a raw q/k/v projection check the projection, its gains
    # and the rotary base before any HIP call, then the decode arguments as the plain views
    L = lib()
    loc = lambda qkv=FAKE, gq=FAKE, gk=FAKE, eps=1e-6, base=1e6, k=None, sinks=4, window=2048, ws=FAKE: \
        L.oda_decode_local_qkv(qkv, gq, gk, eps, base, k or kv(), sinks, window, 0.1, None, 1, FAKE, ws, 1 << 20,
                               None)
    full = lambda qkv=FAKE, gq=FAKE, gk=FAKE, eps=1e-6, base=1e6, k=None, ws=FAKE: \
        L.oda_decode_full_qkv(qkv, gq, gk, eps, base, k or kv(), 0.1, None, 1, FAKE, ws, 1 << 20, None)
    for call in (loc, full):
        assert call(qkv=None) == SK_E_NULL
        assert call(gq=None) == SK_E_NULL
        assert call(gk=None) == SK_E_NULL
        assert call(base=0.0) == SK_E_RANGE
        assert call(base=float("nan")) == SK_E_RANGE
        assert call(eps=-1.0) == SK_E_RANGE
        assert call(k=kv(head_dim=64)) == SK_E_SHAPE
        assert call(k=kv(num_q_heads=12)) == SK_E_HEADS
        assert call(ws=None) == SK_E_NULL
    assert loc(sinks=-1) == SK_E_RANGE
    assert loc(window=0) == SK_E_RANGE


def test_other_entry_points_validation():
    L = lib()
    assert L.oda_recall_score(None, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 0.0, FAKE, FAKE, FAKE, 1 << 20, None) == SK_E_NULL
    assert L.oda_recall_score(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 4, 0.0, FAKE, FAKE, FAKE, 1 << 20, None) == SK_E_RANGE
    assert L.oda_recall_score(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 6, 4, 0.0, FAKE, FAKE, FAKE, 1 << 20, None) == SK_E_RANGE
    assert L.oda_recall_score(FAKE, FAKE, FAKE, FAKE, FAKE, 65, 8, 4, 0.0, FAKE, FAKE, FAKE, 1 << 20, None) == SK_E_RANGE
    assert L.oda_recall_score(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 8, 4, 0.0, FAKE, FAKE, FAKE, 8, None) == SK_E_WORKSPACE
    # the last workgroup stages ceil(hidden / 4) * batch partial sums: 16384 at most
    assert L.oda_recall_score(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 8, 1028, 0.0, FAKE, FAKE, FAKE, 1 << 20, None) == SK_E_RANGE
    assert L.oda_recall_score(FAKE, FAKE, FAKE, FAKE, FAKE, 64, 8, 1024, 0.0, FAKE, FAKE, FAKE, 8, None) == SK_E_WORKSPACE
    assert L.oda_gate_scores(None, 1, 0.0, None, FAKE, None) == SK_E_NULL
    assert L.oda_gate_scores(FAKE, 0, 0.0, None, FAKE, None) == SK_E_RANGE
    assert L.da_keep_mask(None, kv(), 1024, FAKE, None) == SK_E_NULL
    assert L.da_keep_mask(FAKE, kv(), -1, FAKE, None) == SK_E_RANGE
    tags = _lib.DaTagsStruct(5, 6, 7, 100)
    assert L.da_declare(None, FAKE, FAKE, 2, FAKE, tags, kv(), 1024, FAKE, FAKE, None) == SK_E_NULL
    assert L.da_declare(FAKE, FAKE, None, 2, FAKE, tags, kv(), 1024, FAKE, FAKE, None) == SK_E_NULL
    assert L.da_declare(FAKE, FAKE, FAKE, -1, FAKE, tags, kv(), 1024, FAKE, FAKE, None) == SK_E_RANGE
    assert L.da_declare(FAKE, FAKE, None, 0, FAKE, tags, kv(), -1, FAKE, FAKE, None) == SK_E_RANGE
    assert L.da_declare(FAKE, FAKE, None, 0, FAKE, tags, kv(), 1024, None, None, None) == SK_E_NULL  # decl
    # (keep_mask may be NULL: only the declaration is written)
    assert L.da_decode_blocks(FAKE, kv(), None, None, None, FAKE, FAKE, FAKE, 0.1, None, 2, FAKE, FAKE,
                              1 << 30, None) == SK_E_NULL
    assert L.da_gather(kv(), None, FAKE, FAKE, FAKE, None, 2, None, None) == SK_E_NULL
    assert L.da_decode_gathered(FAKE, kv(), None, None, None, FAKE, FAKE, 0.1, None, 2, FAKE, FAKE, 1 << 30,
                                None) == SK_E_NULL
    # dense layers of the weight-bearing step
    assert L.sk_gemv(None, 8, 512, FAKE, 0, None, 1e-6, None, 0, FAKE + 64, None, 0, None) == SK_E_NULL
    assert L.sk_gemv(FAKE, 8, 500, FAKE, 0, None, 1e-6, None, 0, FAKE + 64, None, 0, None) == SK_E_SHAPE
    assert L.sk_gemv(FAKE, 8, 5120, FAKE, 0, None, 1e-6, None, 0, FAKE + 64, None, 0, None) == SK_E_SHAPE
    assert L.sk_gemv(FAKE, 8, 512, FAKE, 1, None, 1e-6, None, 0, FAKE + 64, None, 0, None) == SK_E_NULL
    assert L.sk_gemv(FAKE, 8, 512, FAKE, 0, None, 1e-6, FAKE, 1, FAKE + 64, None, 0, None) == SK_E_RANGE
    assert L.sk_gemv(FAKE, 8, 512, FAKE, 0, None, 1e-6, None, 0, FAKE, None, 0, None) == SK_E_RANGE   # y == x
    assert L.sk_gemv(FAKE, 0, 512, FAKE, 0, None, 1e-6, None, 0, FAKE + 64, None, 0, None) == SK_E_RANGE
    qa = [FAKE] * 5
    assert L.sk_qkv_rope(*qa, 2048, 16, 6, 1e-6, 1e6, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == SK_E_HEADS
    assert L.sk_qkv_rope(*qa, 2000, 16, 8, 1e-6, 1e6, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None) == SK_E_SHAPE
    assert L.sk_qkv_rope(*qa, 2048, 16, 8, 1e-6, 1e6, FAKE, None, FAKE, FAKE, FAKE, None, 0, None) == SK_E_NULL
    assert L.sk_rmsnorm(FAKE, FAKE, 0, 1e-6, FAKE, None, 0, None) == SK_E_RANGE
    assert L.sk_embed(FAKE, 0, 8, FAKE, FAKE, None, None, 0, None) == SK_E_RANGE
    assert L.sk_select(None, 1, FAKE, FAKE, 8, FAKE, None) == SK_E_NULL
    assert L.da_decode_declared(FAKE, kv(), None, None, None, 1024, 0.1, None, 0, FAKE, FAKE, 1 << 20,
                                None) == SK_E_NULL
    assert L.da_decode_declared(FAKE, kv(), None, None, FAKE, -1, 0.1, None, 0, FAKE, FAKE, 1 << 20,
                                None) == SK_E_RANGE
    assert L.sk_stream_read(FAKE, 64, None, None) == SK_E_NULL
    assert L.sk_stream_read(None, 64, FAKE, None) == SK_E_NULL
    assert L.sk_stream_read(FAKE, 24, FAKE, None) == SK_E_RANGE        # not a multiple of 16
    assert L.sk_stream_read(FAKE + 8, 64, FAKE, None) == SK_E_RANGE    # data not 16-byte aligned
    assert L.sk_kv_write(kv(), 1, 0, 1, FAKE, FAKE, None, None) == SK_E_RANGE       # request >= batch
    assert L.sk_kv_write(kv(), 0, 1599, 2, FAKE, FAKE, None, None) == SK_E_RANGE    # past max_blocks*16
    assert L.sk_kv_write(kv(), 0, 0, 1, None, FAKE, None, None) == SK_E_NULL
    assert L.sk_kv_write(kv(), 0, 0, 0, None, None, None, None) == 0  # empty write: nothing enqueued
    assert L.sk_kv_read(kv(), 0, -1, 1, FAKE, FAKE, None, None) == SK_E_RANGE
    assert L.sk_kv_append(kv(), None, FAKE, None, 0, None, None) == SK_E_NULL
    assert L.sk_workspace_init(None, 1 << 20, None) == SK_E_NULL
    assert L.sk_workspace_init(FAKE, 8, None) == SK_E_WORKSPACE
    assert L.sk_workspace_error(None, FAKE, None) == SK_E_NULL


def test_workspace_size_monotone_and_status_strings():
    L = lib()
    prev = 0
    for b in (1, 2, 8, 32, 1024):
        for h in (1, 8, 32):
            s = L.sk_workspace_bytes(b, h)
            assert s > 0
            if h == 32:
                assert s >= prev
                prev = s
    assert L.sk_workspace_bytes(32, 32) >= L.sk_workspace_bytes(1, 32)
    for code in (0, -1, -2, -3, -4, -5, -1001, 7):
        assert isinstance(L.sk_status_str(code), bytes) and L.sk_status_str(code)


def _header_prototypes():
    """name -> list of parameter type strings, parsed from include/sparsekv.h."""
    import re
    text = open(_lib.HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"#.*", " ", text)
    protos = {}
    for m in re.finditer(r"([A-Za-z_][\w\s\*]*?)\b(\w+)\s*\(([^)]*)\)\s*;", text):
        name, params = m.group(2), m.group(3)
        parts = [p.strip() for p in params.split(",") if p.strip()]
        if parts == ["void"]:
            parts = []
        protos[name] = [re.sub(r"\s*\b\w+$", "", p) if not p.endswith("*") else p for p in parts]
    return protos


def _kind_of_c(t):
    t = " ".join(t.replace("const ", "").split())
    if "*" in t or t == "hipStream_t":
        return "ptr"
    return {"int32_t": "i32", "int": "i32", "float": "f32", "size_t": "u64", "uint64_t": "u64",
            "sk_paged_kv": "sk_paged_kv", "sk_da_tags": "sk_da_tags"}[t]


def _kind_of_ctypes(t):
    if t in (ctypes.c_void_p, ctypes.c_char_p):
        return "ptr"
    if t is _lib.PagedKVStruct:
        return "sk_paged_kv"
    if t is _lib.DaTagsStruct:
        return "sk_da_tags"
    if t is ctypes.c_int32:
        return "i32"
    if t is ctypes.c_float:
        return "f32"
    if t in (ctypes.c_size_t, ctypes.c_uint64):
        return "u64"
    raise AssertionError(t)


def test_binding_signatures_match_the_header():
    """Every ctypes signature has the header's parameter count and kinds, in order."""
    protos = _header_prototypes()
    assert set(protos) == set(_lib._SIGNATURES), set(protos) ^ set(_lib._SIGNATURES)
    for name, (_, args) in _lib._SIGNATURES.items():
        want = [_kind_of_c(t) for t in protos[name]]
        got = [_kind_of_ctypes(t) for t in args]
        assert got == want, (name, got, want)


def test_struct_layouts_match_the_header():
    assert ctypes.sizeof(_lib.PagedKVStruct) == 2 * 8 + 2 * 8 + 6 * 4 + 8  # 4 pointers, 6 int32, int64
    assert _lib.PagedKVStruct.num_phys_blocks.offset == 56
    assert ctypes.sizeof(_lib.DaTagsStruct) == 16


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """There is no CPU or PyTorch fallback behind the entry points: with the library
    absent the binding raises LibraryMissing, and host tensors are refused before any
    call (the kernels take device memory only)."""
    import torch
    from sparse_kv_recall_amd import ops
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libsparsekv.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    for fn in (lambda: ops.workspace_bytes(1, 8), lambda: ops.workspace(1, 8, device="cpu"),
               lambda: _lib.call("sk_status_str", 0)):
        with pytest.raises(_lib.LibraryMissing):
            fn()
    for fn in (lambda: ops.PagedKVCache(4, 1, 8, 2, 4, device="cpu"),
               lambda: ops.stream_read(torch.zeros(64, dtype=torch.int32))):
        with pytest.raises(ValueError, match="GPU tensor"):
            fn()
