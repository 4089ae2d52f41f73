"""ctypes loader for libsparsekv.so (the HIP library); argument marshalling only.

There is no fallback: if the library is missing or cannot be loaded, every call
raises. Build it with ``python -m sparse_kv_recall_amd.build`` or
``__graft_entry__.build()``.
"""

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsparsekv.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "sparsekv.h")

c_void_p, c_int32, c_int64, c_float, c_size_t = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                 ctypes.c_float, ctypes.c_size_t)
c_uint64 = ctypes.c_uint64


class PagedKVStruct(ctypes.Structure):
    """Mirror of ``sk_paged_kv`` in include/sparsekv.h."""
    _fields_ = [("k_pool", c_void_p), ("v_pool", c_void_p), ("block_tables", c_void_p),
                ("seq_lens", c_void_p), ("batch", c_int32), ("num_q_heads", c_int32),
                ("num_kv_heads", c_int32), ("head_dim", c_int32), ("block_size", c_int32),
                ("max_blocks", c_int32), ("num_phys_blocks", c_int64)]


class DaTagsStruct(ctypes.Structure):
    """Mirror of ``sk_da_tags`` in include/sparsekv.h."""
    _fields_ = [("global_tag", c_int32), ("focus_tag", c_int32), ("local_tag", c_int32),
                ("segment_base", c_int32)]


_SIGNATURES = {
    "sk_workspace_bytes": (c_size_t, [c_int32, c_int32]),
    "sk_workspace_init": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "sk_workspace_error": (c_int32, [c_void_p, c_void_p, c_void_p]),
    "sk_status_str": (ctypes.c_char_p, [c_int32]),
    "sk_kv_write": (c_int32, [PagedKVStruct, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "sk_kv_read": (c_int32, [PagedKVStruct, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "sk_kv_append": (c_int32, [PagedKVStruct, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "oda_decode_local": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_int32, c_int32, c_float,
                                   c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "oda_decode_full": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                                  c_void_p, c_void_p, c_size_t, c_void_p]),
    "oda_local_tiles_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "oda_local_tiles": (c_int32, [PagedKVStruct, c_int32, c_int32, c_void_p, c_size_t, c_void_p]),
    "oda_decode_local_tiles": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_size_t, c_void_p, c_void_p, c_int32,
                                         c_int32, c_float, c_void_p, c_int32, c_void_p, c_void_p, c_size_t,
                                         c_void_p]),
    "oda_decode_local_qkv": (c_int32, [c_void_p, c_void_p, c_void_p, c_float, c_float, PagedKVStruct, c_int32, c_int32,
                                       c_float, c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "oda_decode_full_qkv": (c_int32, [c_void_p, c_void_p, c_void_p, c_float, c_float, PagedKVStruct, c_float,
                                      c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "oda_decode_full_noalloc": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_float, c_void_p, c_int32,
                                          c_void_p, c_void_p, c_void_p]),
    "oda_recall_score": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                   c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "oda_gate_scores": (c_int32, [c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p]),
    "da_keep_mask": (c_int32, [c_void_p, PagedKVStruct, c_int32, c_void_p, c_void_p]),
    "da_declare": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, DaTagsStruct, PagedKVStruct, c_int32,
                             c_void_p, c_void_p, c_void_p]),
    "sk_gemv": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_float, c_void_p, c_int32,
                          c_void_p, c_void_p, c_int32, c_void_p]),
    "sk_qkv_rope": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_float,
                              c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p]),
    "sk_rmsnorm": (c_int32, [c_void_p, c_void_p, c_int32, c_float, c_void_p, c_void_p, c_int32, c_void_p]),
    "sk_embed": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p]),
    "sk_select": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p]),
    "sk_stream_read": (c_int32, [c_void_p, c_uint64, c_void_p, c_void_p]),
    "da_decode_declared": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                     c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "da_gather": (c_int32, [PagedKVStruct, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                            c_void_p]),
    "da_decode_gathered": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_float, c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "oda_decode_views": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_int32, c_int32, c_float, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "da_decode_blocks": (c_int32, [c_void_p, PagedKVStruct, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_float, c_void_p, c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
}

_lib = None


class LibraryMissing(RuntimeError):
    pass


def load():
    """Load (once) and return the ctypes handle of libsparsekv.so."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryMissing("%s is not built; run `python -m sparse_kv_recall_amd.build` "
                             "(or __graft_entry__.build()) first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions():
    """Names of the functions declared in include/sparsekv.h."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "for", "switch", "return", "sizeof")))


class SKError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        msg = load().sk_status_str(status).decode()
        super().__init__("%s failed with status %d (%s)" % (fn, status, msg))


def call(name, *args):
    st = getattr(load(), name)(*args)
    if st != 0:
        raise SKError(name, st)
    return st
