"""ctypes binding of synth/libsk_synth.so: device fills of the synthetic streams and the
per-step feed kernel. Outputs are bit-identical to synth.rng on the host."""

import ctypes
import os

import numpy as np
import torch

from . import rng
from .workloads import C_K, C_Q, C_SCORE, C_V, C_X

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsk_synth.so")
_lib = None

vp, i32, i64, u64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float


def load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("%s is not built; run `python -m synth.build`" % LIB_PATH)
        lib = ctypes.CDLL(LIB_PATH)
        lib.synth_fill_f32.argtypes = [vp, i64, u64, i64, f32, vp]
        lib.synth_fill_bf16.argtypes = [vp, i64, u64, i64, f32, vp]
        lib.synth_feed.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, u64, u64, u64, u64, u64, f32,
                                   vp, vp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
        lib.synth_set_step.argtypes = [vp, i32, vp]
        for f in (lib.synth_fill_f32, lib.synth_fill_bf16, lib.synth_feed, lib.synth_set_step):
            f.restype = i32
        _lib = lib
    return _lib


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ok(st, name):
    if st != 0:
        raise RuntimeError("%s failed with status %d" % (name, st))


def fill_normal_(out, key, index0, sigma=1.0):
    """Fill a float32 or bfloat16 GPU tensor with stream values index0 .. index0+numel-1."""
    scale = float(rng.unit_scale(sigma))
    if out.dtype == torch.float32:
        _ok(load().synth_fill_f32(out.data_ptr(), out.numel(), key, int(index0), scale, _stream(out)), "fill_f32")
    elif out.dtype == torch.bfloat16:
        _ok(load().synth_fill_bf16(out.data_ptr(), out.numel(), key, int(index0), scale, _stream(out)), "fill_bf16")
    else:
        raise ValueError("unsupported dtype %s" % out.dtype)
    return out


class Feeder:
    """Fixed per-step input buffers of a workload plus the feed kernel that fills them.

    After ``step()`` the buffers hold step t's inputs (t = internal counter modulo the
    workload's step count) and seq_lens = H0 + t + 1; the counter then advances.
    The launch reads its step index from device memory, so it can be captured once in
    a HIP graph and replayed every step.
    """

    def __init__(self, wl, seq_lens, device="cuda", with_x=False, with_scores=False, with_decl=False,
                 with_tokens=False):
        self.wl = wl
        dev = torch.device(device)
        L, P, B = wl.layers, wl.passes, wl.batch
        self.state = torch.zeros(2, dtype=torch.int32, device=dev)
        self.seq_lens = seq_lens
        self.H0 = torch.as_tensor(np.asarray(wl.H0, dtype=np.int32), device=dev)
        self.q = torch.empty((L, P, B, wl.Hq, 128), dtype=torch.float32, device=dev)
        self.k = torch.empty((L, P, B, wl.Hkv, 128), dtype=torch.bfloat16, device=dev)
        self.v = torch.empty_like(self.k)
        self.x = torch.empty((B, wl.x_dim), dtype=torch.float32, device=dev) if with_x else None
        self.scores = torch.empty(B, dtype=torch.float32, device=dev) if with_scores else None
        self.sched = (torch.as_tensor(wl.sched_scores.astype(np.float32), device=dev)
                      if (with_scores and wl.sched_scores is not None) else None)
        self.decl_table = (torch.as_tensor(wl.decl.astype(np.int32), device=dev) if with_decl else None)
        self.decl = torch.empty((B, 4), dtype=torch.int32, device=dev) if with_decl else None
        self.token_table = (torch.as_tensor(wl.tokens.astype(np.int32), device=dev) if with_tokens else None)
        self.tokens = torch.empty(B, dtype=torch.int32, device=dev) if with_tokens else None

    def _p(self, t):
        return 0 if t is None else t.data_ptr()

    def step(self):
        wl = self.wl
        _ok(load().synth_feed(self.state.data_ptr(), self.seq_lens.data_ptr(), self.H0.data_ptr(), wl.batch,
                              wl.layers, wl.passes, wl.Hq, wl.Hkv, wl.steps, wl.key(C_Q), wl.key(C_K),
                              wl.key(C_V), wl.key(C_X), wl.key(C_SCORE), float(rng.unit_scale()),
                              self.q.data_ptr(), self.k.data_ptr(), self.v.data_ptr(), wl.x_dim,
                              self._p(self.x), self._p(self.sched), self._p(self.scores), self._p(self.decl_table),
                              self._p(self.decl), self._p(self.token_table), self._p(self.tokens),
                              _stream(self.state)), "synth_feed")

    def set_step(self, t):
        _ok(load().synth_set_step(self.state.data_ptr(), int(t), _stream(self.state)), "synth_set_step")
