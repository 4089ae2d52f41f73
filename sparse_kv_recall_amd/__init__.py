"""MI355X-native selectively-read decode attention (ODA local/full views, DA keep-lists).

The computation lives in libsparsekv.so (HIP for gfx950, C ABI in include/sparsekv.h);
``sparse_kv_recall_amd.ops`` is its torch-facing binding. Importing this package loads
nothing; the library is loaded on first use and a missing library raises.
"""

__all__ = ["ops"]
