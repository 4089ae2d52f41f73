"""GPU parity of oda_decode_views, the per-request views of a batch in one launch: each
running request against the fp64 oracle for its view (Full, Local, or its gathered block
list), with fused commits; requests whose view value names no view keep their output rows
and their slot n-1. Batches of 12 and 64 (per-wave planning), 65 and 100 (workgroup
planning), 256 (the largest batch ranked for the balanced order) and 257 (workgroup order). With equal lengths and one view for every request the plan and the tile order
are those of the single-view launch, so the outputs are bit-identical to it."""

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, keysets
from synth import rng
from tests.helpers import (SCALE, HostCache, bf16_tensor_to_bits, bits_to_bf16_tensor, check_close, check_tight,
                           rand_bits, rand_f32, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _mask_words(kept_per_req, max_blocks):
    words = np.zeros((len(kept_per_req), (max_blocks + 31) // 32), np.uint32)
    for b, kept in enumerate(kept_per_req):
        for blk in kept:
            words[b, blk // 32] |= np.uint32(1 << (blk % 32))
    return words


@pytest.mark.parametrize("B,sinks,window,Hq,Hkv", [(12, 4, 2048, 16, 4), (64, 4, 2048, 16, 4), (65, 4, 300, 16, 4),
                                                   (100, 3, 40, 16, 4), (12, 4, 2048, 32, 2), (70, 4, 500, 32, 2),
                                                   (40, 4, 2048, 15, 3), (90, 4, 500, 10, 5), (20, 4, 2048, 16, 16)])
def test_views_one_launch(B, sinks, window, Hq, Hkv):
    # query groups of 4 and of 16 (the merge then works on four output elements per thread);
    # 3, 5 and 16 KV heads, whose split slots per KV head leave a remainder of the grid, the
    # 90-request batch through the workgroup plan and its ranking for the balanced order
    g = np.random.default_rng(90 + B + Hkv)
    ns = [int(x) for x in g.integers(1, 6000, size=B)]
    ns[:5] = [1, 16, 17, 2052, 5999]
    _views_case(g, B, ns, sinks, window, Hq, Hkv)


@pytest.mark.parametrize("B", [256, 257])
def test_views_balanced_order_batch_bound(B):
    # 256 requests: the largest batch ranked in LDS for the balanced order; 257: the plain
    # workgroup order. Log-uniform lengths 1..1500, so the long requests take several splits.
    g = np.random.default_rng(80 + B)
    ns = [int(x) for x in np.floor(np.exp(g.uniform(0.0, np.log(1500), size=B)))]
    ns[:5] = [1, 16, 17, 1500, 1499]
    _views_case(g, B, ns, 4, 300, 8, 2, drop_last_every=3)


def _views_case(g, B, ns, sinks, window, Hq, Hkv, drop_last_every=0):
    # drop_last_every = k: every k-th request's kept blocks leave out the block of position
    # n-1, so its list view does not attend the current token but still commits it
    from sparse_kv_recall_amd import ops
    hc = HostCache(Hq, Hkv, ns, seed=91)
    # views: 0 Local, 1 Full, 2 blocks, 5 none (the request does not run)
    view = g.choice([0, 1, 2, 5], size=B, p=[0.3, 0.3, 0.3, 0.1]).astype(np.int32)
    view[:4] = [0, 1, 2, 5]
    kept = []
    for b, n in enumerate(ns):
        nb = (n + 15) // 16
        ks = set(g.choice(nb, size=max(1, nb // 4), replace=False).tolist()) | {nb - 1}
        if drop_last_every and b % drop_last_every == 1 and nb > 1:
            ks = (ks - {nb - 1}) or {0}
        kept.append(sorted(ks))
    mask = torch.as_tensor(_mask_words(kept, hc.max_blocks).view(np.int32), device="cuda")
    q = rand_f32(rng.mix_key(992, B), (B, Hq, 128), 1.0)
    kn = rand_bits(rng.mix_key(993, B, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(993, B, 2), B, Hkv)
    vt = torch.as_tensor(view, device="cuda")
    gat = torch.zeros((B, hc.max_blocks), dtype=torch.int32, device="cuda")
    cnt = torch.zeros_like(gat)
    num = torch.zeros(B, dtype=torch.int32, device="cuda")
    ws = ops.workspace(B, Hq)
    ops.da_gather(hc.kv, mask, gathered=gat, gathered_cnt=cnt, num_kept=num, sel=vt, sel_value=ops.MODE_BLOCKS,
                  ws=ws)
    out = torch.full((B, Hq, 128), 7.0, device="cuda")
    ops.oda_decode_views(torch.as_tensor(q, device="cuda"), hc.kv, vt, gat, cnt, num, bits_to_bf16_tensor(kn),
                         bits_to_bf16_tensor(vn), sinks=sinks, window=window, out=out, ws=ws)
    got = out.cpu().numpy()
    assert ops.workspace_error(ws) == 0
    for b, n in enumerate(ns):
        kr, vr = ops.kv_read(hc.kv, b, n - 1, 1)
        if view[b] not in (0, 1, 2):
            assert (got[b] == 7.0).all(), b
            assert np.array_equal(bf16_tensor_to_bits(kr)[0], hc.k[b][n - 1]), b
            assert np.array_equal(bf16_tensor_to_bits(vr)[0], hc.v[b][n - 1]), b
            continue
        k, v = hc.k[b].copy(), hc.v[b].copy()
        oracle.oda.commit(k, v, n, kn[b], vn[b])
        keys = (keysets.local_keys(n, sinks, window), keysets.full_keys(n), keysets.block_keys(n, kept[b]))[view[b]]
        ref = attention.attend(q[b], k, v, keys, SCALE)
        # a row over a few keys (n = 4) is not averaged down: the error model's bound
        check_tight(got[b], ref, q[b], k, v, keys, SCALE, what="b=%d n=%d view=%d" % (b, n, view[b]))
        assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b]) and np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b])


def test_views_none_running():
    # no request names a view: every workgroup leaves at once, nothing is written
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    ns = [300, 5000, 17]
    hc = HostCache(Hq, Hkv, ns, seed=95)
    q = torch.as_tensor(rand_f32(rng.mix_key(995), (3, Hq, 128), 1.0), device="cuda")
    vt = torch.full((3,), 9, dtype=torch.int32, device="cuda")
    gat = torch.zeros((3, hc.max_blocks), dtype=torch.int32, device="cuda")
    out = torch.full((3, Hq, 128), 7.0, device="cuda")
    ops.oda_decode_views(q, hc.kv, vt, gat, torch.zeros_like(gat), torch.zeros(3, dtype=torch.int32, device="cuda"),
                         out=out)
    assert (out.cpu().numpy() == 7.0).all()


@pytest.mark.parametrize("view", [0, 1, 2])
def test_views_single_view_bit_identical(view):
    from sparse_kv_recall_amd import ops
    Hq, Hkv, B, n = 32, 8, 6, 9000
    hc_v = HostCache(Hq, Hkv, [n] * B, seed=96)
    hc_s = HostCache(Hq, Hkv, [n] * B, seed=96)
    nb = (n + 15) // 16
    kept = [list(range(0, nb, 3)) + [nb - 1]] * B
    mask = torch.as_tensor(_mask_words(kept, hc_v.max_blocks).view(np.int32), device="cuda")
    q = torch.as_tensor(rand_f32(rng.mix_key(996, view), (B, Hq, 128), 1.0), device="cuda")
    kt = bits_to_bf16_tensor(rand_bits(rng.mix_key(997, 1), B, Hkv))
    vt = bits_to_bf16_tensor(rand_bits(rng.mix_key(997, 2), B, Hkv))
    sel = torch.full((B,), view, dtype=torch.int32, device="cuda")
    lists = []
    for hc in (hc_v, hc_s):
        gat = torch.zeros((B, hc.max_blocks), dtype=torch.int32, device="cuda")
        cnt, num = torch.zeros_like(gat), torch.zeros(B, dtype=torch.int32, device="cuda")
        ops.da_gather(hc.kv, mask, gathered=gat, gathered_cnt=cnt, num_kept=num)
        lists.append((gat, cnt, num))
    got = ops.oda_decode_views(q, hc_v.kv, sel, *lists[0], k_new=kt, v_new=vt)
    if view == ops.MODE_LOCAL:
        ref = ops.oda_decode_local(q, hc_s.kv, kt, vt)
    elif view == ops.MODE_FULL:
        ref = ops.oda_decode_full(q, hc_s.kv, kt, vt)
    else:
        ref = ops.da_decode_gathered(q, hc_s.kv, *lists[1], k_new=kt, v_new=vt)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), ref.cpu().numpy().view(np.uint32))
    kv_, vv_ = ops.kv_read(hc_v.kv, 0, n - 1, 1)
    ks_, vs_ = ops.kv_read(hc_s.kv, 0, n - 1, 1)
    assert np.array_equal(bf16_tensor_to_bits(kv_), bf16_tensor_to_bits(ks_))
    assert np.array_equal(bf16_tensor_to_bits(vv_), bf16_tensor_to_bits(vs_))
