"""GPU test of the allocation-free Full view (oda_decode_full_noalloc) through the C ABI.

It runs the same kernels as oda_decode_full with the split tickets and partials in the
library's device array instead of a caller workspace, so its outputs and commits must
equal oda_decode_full's bit for bit. Two calls in a row, the second on a smaller input,
so the second one reuses the array the first left behind; a third call under a gate of
zeros must leave the output untouched.
"""

import numpy as np
import pytest
import torch

from oracle import attention, keysets
from synth import rng
from tests.helpers import SCALE, HostCache, bf16_tensor_to_bits, bits_to_bf16_tensor, check_close, rand_bits, \
    rand_f32, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _case(Hq, Hkv, ns, seed):
    hc = HostCache(Hq, Hkv, ns, seed=seed)
    B = len(ns)
    q = torch.as_tensor(rand_f32(rng.mix_key(950, seed, 0), (B, Hq, 128)), device="cuda")
    kn = rand_bits(rng.mix_key(950, seed, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(950, seed, 2), B, Hkv)
    return hc, q, kn, vn


def _slots(hc):
    from sparse_kv_recall_amd import ops
    ks, vs = [], []
    for b, n in enumerate(hc.ns):
        k, v = ops.kv_read(hc.kv, b, n - 1, 1)
        ks.append(bf16_tensor_to_bits(k)[0])
        vs.append(bf16_tensor_to_bits(v)[0])
    return np.stack(ks), np.stack(vs)


def test_noalloc_full_equals_workspace_full_twice():
    from sparse_kv_recall_amd import ops
    print("noalloc: call 1 (batch 3, 32/8 heads, n = 9000, 777, 40001)", flush=True)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    cases = [(32, 8, [9000, 777, 40001], 71), (16, 8, [1203], 72)]  # the second call is smaller
    for i, (Hq, Hkv, ns, seed) in enumerate(cases):
        if i:
            print("noalloc: call 2 (batch 1, 16/8 heads, n = 1203)", flush=True)
        hc, q, kn, vn = _case(Hq, Hkv, ns, seed)
        knt, vnt = bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn)
        out_ref = ops.oda_decode_full(q, hc.kv, knt, vnt)
        torch.cuda.synchronize()
        k_ref, v_ref = _slots(hc)
        # restore the slots the first call committed, so the second commit is observable
        for b, n in enumerate(ns):
            ops.kv_write(hc.kv, b, n - 1, bits_to_bf16_tensor(hc.k[b][n - 1:n]), bits_to_bf16_tensor(hc.v[b][n - 1:n]))
        out = torch.full_like(out_ref, float("nan"))
        ops.oda_decode_full_noalloc(q, hc.kv, out, knt, vnt, dev_err=err)
        torch.cuda.synchronize()
        assert torch.equal(out, out_ref), "call %d differs from oda_decode_full" % (i + 1)
        k_got, v_got = _slots(hc)
        assert np.array_equal(k_got, k_ref) and np.array_equal(v_got, v_ref)
        assert np.array_equal(k_got, kn) and np.array_equal(v_got, vn)
        assert int(err.item()) == 0
        # and against the fp64 oracle (the committed token is the current one)
        got = out.cpu().numpy()
        qh = q.cpu().numpy()
        for b, n in enumerate(ns):
            kb, vb = hc.k[b].copy(), hc.v[b].copy()
            kb[n - 1], vb[n - 1] = kn[b], vn[b]
            ref = attention.attend(qh[b], kb, vb, keysets.full_keys(n), SCALE)
            check_close(got[b], ref, what="noalloc call %d n=%d" % (i + 1, n))
    # a gate of zeros: nothing runs, the output keeps its contents
    print("noalloc: call 3 (gated off)", flush=True)
    hc, q, kn, vn = _case(32, 8, [5000], 73)
    out = torch.full((1, 32, 128), 7.0, device="cuda")
    sel = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.oda_decode_full_noalloc(q, hc.kv, out, sel=sel, sel_value=1, dev_err=err)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


def test_noalloc_rejects_oversized_batch():
    from sparse_kv_recall_amd import _lib, ops
    hc, q, _, _ = _case(32, 8, [100], 74)
    big = ops.PagedKVCache(hc.kv.num_phys_blocks, 600, 32, 8, hc.kv.max_blocks)
    qb = torch.zeros((600, 32, 128), device="cuda")
    out = torch.zeros_like(qb)
    with pytest.raises(_lib.SKError) as e:
        ops.oda_decode_full_noalloc(qb, big, out)
    assert e.value.status == -5
