"""GPU parity of the decode entry points against the fp64 oracle on small shapes.

Shapes span several 16-position tiles, several splits and ragged tails; unwritten
slots and unkept blocks of the pool hold bf16 NaN, so any over-read shows up.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, gather, keysets
from synth import rng
from tests.helpers import (SCALE, HostCache, bf16_tensor_to_bits, bits_to_bf16_tensor, check_close, check_tight,
                           rand_bits, rand_f32, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]

NS_EDGE = [1, 3, 4, 5, 15, 16, 17, 31, 32, 33, 47, 100, 2051, 2052, 2053, 2069, 4097]


def _q(Hq, B, seed, sigma=1.0):
    return rand_f32(rng.mix_key(901, seed), (B, Hq, 128), sigma)


def _run_full(hc, q, **kw):
    from sparse_kv_recall_amd import ops
    out = ops.oda_decode_full(torch.as_tensor(q, device="cuda"), hc.kv, **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (16, 8), (32, 8), (4, 4), (32, 2)])
def test_full_edge_lengths(Hq, Hkv):
    ns = NS_EDGE if Hq <= 16 else NS_EDGE[::2]
    hc = HostCache(Hq, Hkv, ns, seed=Hq + Hkv)
    q = _q(Hq, len(ns), seed=3)
    got = _run_full(hc, q)
    for b, n in enumerate(ns):
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
        check_close(got[b], ref, what="full n=%d" % n)
        if n <= 5000:
            check_tight(got[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE, what="full tight n=%d" % n)


@pytest.mark.parametrize("sinks,window", [(4, 2048), (3, 20), (0, 17), (20, 5), (4, 1)])
def test_local_edge_lengths(sinks, window):
    Hq, Hkv = 8, 2
    ns = NS_EDGE
    hc = HostCache(Hq, Hkv, ns, seed=sinks * 31 + window)
    q = _q(Hq, len(ns), seed=4)
    from sparse_kv_recall_amd import ops
    out = ops.oda_decode_local(torch.as_tensor(q, device="cuda"), hc.kv, sinks=sinks, window=window)
    got = out.cpu().numpy()
    for b, n in enumerate(ns):
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.local_keys(n, sinks, window), SCALE)
        check_tight(got[b], ref, q[b], hc.k[b], hc.v[b], keysets.local_keys(n, sinks, window), SCALE,
                    what="local n=%d s=%d w=%d" % (n, sinks, window))


def test_local_equals_full_up_to_s_plus_w():
    Hq, Hkv = 8, 2
    ns = [1, 4, 5, 2048, 2052]
    hc = HostCache(Hq, Hkv, ns, seed=77)
    q = _q(Hq, len(ns), seed=5)
    from sparse_kv_recall_amd import ops
    qt = torch.as_tensor(q, device="cuda")
    a = ops.oda_decode_local(qt, hc.kv).cpu().numpy()
    f = ops.oda_decode_full(qt, hc.kv).cpu().numpy()
    for b, n in enumerate(ns):
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
        check_tight(a[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
        check_tight(f[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)


def test_peaky_queries_rescale_path():
    # q scaled x8 plus planted matching keys far apart: the running max changes across splits
    Hq, Hkv = 32, 8
    ns = [5000, 70000]
    hc = HostCache(Hq, Hkv, ns, seed=8, poison=False)
    q = _q(Hq, len(ns), seed=6, sigma=8.0)
    from sparse_kv_recall_amd import ops
    for b, n in enumerate(ns):
        for pos in (3, n // 3, n - 2):
            g = 1
            kb = hc.k[b][pos].copy()
            qk = np.clip(q[b, g * 4] / 8.0, -3, 3)
            kb[g] = oracle_bits(qk)
            hc.k[b][pos] = kb
            ops.kv_write(hc.kv, b, pos, bits_to_bf16_tensor(kb[None]), bits_to_bf16_tensor(hc.v[b][pos][None]))
    got = _run_full(hc, q)
    for b, n in enumerate(ns):
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
        check_close(got[b], ref, what="peaky n=%d" % n)
        check_tight(got[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE, what="peaky tight n=%d" % n)


def oracle_bits(x):
    from synth.rng import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(x, np.float32))


def test_fused_commit_full_and_local():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 16, 8
    ns = [1, 16, 17, 300, 2100]
    hc = HostCache(Hq, Hkv, ns, seed=12)
    B = len(ns)
    q = _q(Hq, B, seed=9)
    kn = rand_bits(rng.mix_key(902, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(902, 2), B, Hkv)
    knt, vnt = bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn)
    qt = torch.as_tensor(q, device="cuda")
    for mode in ("local", "full"):
        if mode == "local":
            out = ops.oda_decode_local(qt, hc.kv, knt, vnt)
        else:
            out = ops.oda_decode_full(qt, hc.kv, knt, vnt)
        got = out.cpu().numpy()
        for b, n in enumerate(ns):
            k = hc.k[b].copy()
            v = hc.v[b].copy()
            oracle.oda.commit(k, v, n, kn[b], vn[b])
            keys = keysets.local_keys(n) if mode == "local" else keysets.full_keys(n)
            ref = attention.attend(q[b], k, v, keys, SCALE)
            check_tight(got[b], ref, q[b], k, v, keys, SCALE, what="%s commit n=%d" % (mode, n))
            kr, vr = ops.kv_read(hc.kv, b, n - 1, 1)
            assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b])
            assert np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b])
            # the rest of the history is untouched
            kr, vr = ops.kv_read(hc.kv, b, 0, n - 1)
            assert np.array_equal(bf16_tensor_to_bits(kr), hc.k[b][:n - 1])
            assert np.array_equal(bf16_tensor_to_bits(vr), hc.v[b][:n - 1])


def test_selector_and_gate_skip_requests():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    ns = [40, 500, 3000, 9]
    hc = HostCache(Hq, Hkv, ns, seed=13)
    B = len(ns)
    q = _q(Hq, B, seed=10)
    qt = torch.as_tensor(q, device="cuda")
    gate = torch.tensor([1, 0, 1, 0], dtype=torch.int32, device="cuda")
    kn = rand_bits(rng.mix_key(903, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(903, 2), B, Hkv)
    out = torch.full((B, Hq, 128), 7.0, device="cuda")
    ops.oda_decode_full(qt, hc.kv, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), sel=gate, sel_value=1, out=out)
    got = out.cpu().numpy()
    for b, n in enumerate(ns):
        if b in (1, 3):
            assert (got[b] == 7.0).all()
            kr, _ = ops.kv_read(hc.kv, b, n - 1, 1)
            assert np.array_equal(bf16_tensor_to_bits(kr)[0], hc.k[b][n - 1])  # nothing committed
        else:
            k = hc.k[b].copy()
            v = hc.v[b].copy()
            oracle.oda.commit(k, v, n, kn[b], vn[b])
            ref = attention.attend(q[b], k, v, keysets.full_keys(n), SCALE)
            check_tight(got[b], ref, q[b], k, v, keysets.full_keys(n), SCALE)


def _mask_words(kept_lists, max_blocks):
    words = (max_blocks + 31) // 32
    m = np.zeros((len(kept_lists), words), np.uint32)
    for b, kept in enumerate(kept_lists):
        for blk in kept:
            m[b, blk // 32] |= np.uint32(1 << (blk % 32))
    return m


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_blocks_gather_and_attention(seed):
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    g = np.random.default_rng(seed)
    ns = [int(x) for x in g.integers(1, 6000, size=5)] + [16, 17, 1]
    hc = HostCache(Hq, Hkv, ns, seed=20 + seed)
    B = len(ns)
    kept = []
    for n in ns:
        nb = (n + 15) // 16
        k = set(g.choice(nb, size=int(g.integers(1, nb + 1)), replace=False).tolist())
        k.add(nb - 1)
        kept.append(sorted(k))
    # stale bits beyond ceil(n/16) must be ignored
    mask = _mask_words([kp + [hc.max_blocks - 1] for kp in kept], hc.max_blocks)
    q = _q(Hq, B, seed=11)
    out, gat, cnt, num = ops.da_decode_blocks(torch.as_tensor(q, device="cuda"), hc.kv,
                                              torch.as_tensor(mask.view(np.int32), device="cuda"))
    got, gat, cnt, num = out.cpu().numpy(), gat.cpu().numpy(), cnt.cpu().numpy(), num.cpu().numpy()
    for b, n in enumerate(ns):
        phys, c = gather.gather_blocks(hc.bt[b], kept[b], n)
        assert num[b] == len(phys)
        assert np.array_equal(gat[b, :num[b]], phys)
        assert np.array_equal(cnt[b, :num[b]], c)
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.block_keys(n, kept[b]), SCALE)
        check_tight(got[b], ref, q[b], hc.k[b], hc.v[b], keysets.block_keys(n, kept[b]), SCALE,
                    what="blocks n=%d" % n)


def test_blocks_all_kept_equals_full_and_commit_when_unkept():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    ns = [1000, 33, 4097]
    hc = HostCache(Hq, Hkv, ns, seed=31)
    B = len(ns)
    q = _q(Hq, B, seed=12)
    qt = torch.as_tensor(q, device="cuda")
    allm = _mask_words([list(range((n + 15) // 16)) for n in ns], hc.max_blocks)
    o_b, _, _, _ = ops.da_decode_blocks(qt, hc.kv, torch.as_tensor(allm.view(np.int32), device="cuda"))
    o_f = ops.oda_decode_full(qt, hc.kv)
    for b, n in enumerate(ns):
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
        check_tight(o_b.cpu().numpy()[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
        check_tight(o_f.cpu().numpy()[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(n), SCALE)
    # keep-list without the current token's block: the token is committed, not attended
    kn = rand_bits(rng.mix_key(904, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(904, 2), B, Hkv)
    kept = [[0, 1], [0], [3, 100]]
    m = _mask_words(kept, hc.max_blocks)
    out, _, _, _ = ops.da_decode_blocks(qt, hc.kv, torch.as_tensor(m.view(np.int32), device="cuda"),
                                        bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn))
    for b, n in enumerate(ns):
        k = hc.k[b].copy()
        v = hc.v[b].copy()
        oracle.oda.commit(k, v, n, kn[b], vn[b])
        ref = attention.attend(q[b], k, v, keysets.block_keys(n, kept[b]), SCALE)
        check_tight(out.cpu().numpy()[b], ref, q[b], k, v, keysets.block_keys(n, kept[b]), SCALE)
        kr, vr = ops.kv_read(hc.kv, b, n - 1, 1)
        assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b])
        assert np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b])


def test_gather_once_decode_per_layer():
    # one block-table rewrite serves several layers: da_gather + da_decode_gathered give
    # exactly what da_decode_blocks gives for each layer's query
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    g = np.random.default_rng(41)
    ns = [5000, 700, 16]
    hc = HostCache(Hq, Hkv, ns, seed=42)
    kept = [sorted(set(g.choice((n + 15) // 16, size=max(1, (n + 15) // 64), replace=False).tolist())) for n in ns]
    mask = torch.as_tensor(_mask_words(kept, hc.max_blocks).view(np.int32), device="cuda")
    gat, cnt, num = ops.da_gather(hc.kv, mask)
    for layer in range(3):
        q = _q(Hq, len(ns), seed=50 + layer)
        qt = torch.as_tensor(q, device="cuda")
        o1 = ops.da_decode_gathered(qt, hc.kv, gat, cnt, num)
        o2, g2, c2, n2 = ops.da_decode_blocks(qt, hc.kv, mask)
        assert torch.equal(o1, o2) and torch.equal(gat, g2) and torch.equal(cnt, c2) and torch.equal(num, n2)
        for b, n in enumerate(ns):
            ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.block_keys(n, kept[b]), SCALE)
            check_tight(o1.cpu().numpy()[b], ref, q[b], hc.k[b], hc.v[b], keysets.block_keys(n, kept[b]), SCALE)


def test_gathered_list_with_bad_block_id():
    # a caller-built list naming a block outside the pool: error bit, that entry attends nothing
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    ns = [300]
    hc = HostCache(Hq, Hkv, ns, seed=43)
    mb = hc.max_blocks
    gat = torch.zeros((1, mb), dtype=torch.int32, device="cuda")
    cnt = torch.zeros_like(gat)
    blocks = [0, 3, 7]
    gat[0, :3] = torch.as_tensor([int(hc.bt[0][0]), 10 ** 6, int(hc.bt[0][7])], dtype=torch.int32)
    cnt[0, :3] = torch.as_tensor([16, 16, 16], dtype=torch.int32)
    num = torch.full((1,), 3, dtype=torch.int32, device="cuda")
    q = _q(Hq, 1, seed=13)
    ws = ops.workspace(1, Hq)
    out = ops.da_decode_gathered(torch.as_tensor(q, device="cuda"), hc.kv, gat, cnt, num, ws=ws)
    assert ops.workspace_error(ws) & 1  # SK_DEVERR_BLOCK_ID
    keys = keysets.block_keys(300, [blocks[0], blocks[2]])
    ref = attention.attend(q[0], hc.k[0], hc.v[0], keys, SCALE)
    check_tight(out.cpu().numpy()[0], ref, q[0], hc.k[0], hc.v[0], keys, SCALE)


def test_large_batch_all_views_with_selector():
    # batches above 64 take the workgroup (LDS) planning path: Full, Local and block
    # lists with a per-request selector and fused commits, 100 ragged requests
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    g = np.random.default_rng(61)
    B = 100
    ns = [int(x) for x in g.integers(1, 2600, size=B)]
    ns[:4] = [1, 16, 17, 2500]
    hc = HostCache(Hq, Hkv, ns, seed=62)
    q = _q(Hq, B, seed=63)
    qt = torch.as_tensor(q, device="cuda")
    view = g.integers(0, 3, size=B).astype(np.int32)  # 0 local, 1 full, 2 blocks
    kept = []
    for n in ns:
        nb = (n + 15) // 16
        kept.append(sorted(set(g.choice(nb, size=max(1, nb // 3), replace=False).tolist()) | {nb - 1}))
    mask = torch.as_tensor(_mask_words(kept, hc.max_blocks).view(np.int32), device="cuda")
    kn = rand_bits(rng.mix_key(905, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(905, 2), B, Hkv)
    kt, vt = bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn)
    sel = torch.as_tensor(view, device="cuda")
    out = torch.full((B, Hq, 128), 7.0, device="cuda")
    ops.oda_decode_local(qt, hc.kv, kt, vt, sinks=4, window=64, sel=sel, sel_value=0, out=out)
    ops.oda_decode_full(qt, hc.kv, kt, vt, sel=sel, sel_value=1, out=out)
    ops.da_decode_blocks(qt, hc.kv, mask, kt, vt, sel=sel, sel_value=2, out=out)
    got = out.cpu().numpy()
    for b, n in enumerate(ns):
        k, v = hc.k[b].copy(), hc.v[b].copy()
        oracle.oda.commit(k, v, n, kn[b], vn[b])
        keys = (keysets.local_keys(n, 4, 64), keysets.full_keys(n), keysets.block_keys(n, kept[b]))[view[b]]
        ref = attention.attend(q[b], k, v, keys, SCALE)
        check_tight(got[b], ref, q[b], k, v, keys, SCALE, what="b=%d n=%d view=%d" % (b, n, view[b]))
        kr, vr = ops.kv_read(hc.kv, b, n - 1, 1)
        assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b]) and np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b])


@pytest.mark.parametrize("B,n_max", [(80, 20000), (256, 1500), (257, 1500)])
def test_large_ragged_batch_balanced_order(B, n_max):
    # above 64 requests with ragged lengths (log-uniform 16..n_max): the workgroup plan splits
    # the long requests too and runs the items in the balanced order (full-size splits, then
    # last splits largest first, grid rounds alternating direction); every request's output
    # and commit against the oracle, so a split run twice or not at all would show. 256
    # requests is the largest batch ranked in LDS for that order; 257 run in workgroup order.
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    g = np.random.default_rng(67)
    ns = [int(x) for x in np.floor(np.exp(g.uniform(np.log(16), np.log(n_max), size=B)))]
    ns[:3] = [n_max, 1, 17]
    hc = HostCache(Hq, Hkv, ns, seed=68)
    q = _q(Hq, B, seed=69)
    kn = rand_bits(rng.mix_key(906, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(906, 2), B, Hkv)
    out = ops.oda_decode_full(torch.as_tensor(q, device="cuda"), hc.kv, bits_to_bf16_tensor(kn),
                              bits_to_bf16_tensor(vn)).cpu().numpy()
    for b, n in enumerate(ns):
        k, v = hc.k[b].copy(), hc.v[b].copy()
        oracle.oda.commit(k, v, n, kn[b], vn[b])
        keys = keysets.full_keys(n)
        ref = attention.attend(q[b], k, v, keys, SCALE)
        check_tight(out[b], ref, q[b], k, v, keys, SCALE, what="b=%d n=%d" % (b, n))
        kr, vr = ops.kv_read(hc.kv, b, n - 1, 1)
        assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b]) and np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b])


@pytest.mark.parametrize("B", [128, 129])
def test_ticket_stride_boundary(B):
    # Split tickets sit 16 words apart while the launch's (request, KV head) pairs fit the
    # ticket region that way (up to 1024 pairs), one word apart beyond. 128 requests at 8 KV
    # heads are exactly 1024 pairs, 129 are past it. The last requests are the longest, so
    # they take several splits and the highest ticket counters; every output and commit is
    # checked against the oracle, and a second launch on the same workspace checks that the
    # counters were left at zero.
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    g = np.random.default_rng(300 + B)
    ns = [int(x) for x in np.floor(np.exp(g.uniform(np.log(16), np.log(1200), size=B)))]
    ns[-3:] = [5000, 3001, 2100]
    hc = HostCache(Hq, Hkv, ns, seed=301)
    q = _q(Hq, B, seed=302)
    kn = rand_bits(rng.mix_key(907, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(907, 2), B, Hkv)
    ws = ops.workspace(B, Hq)
    qt = torch.as_tensor(q, device="cuda")
    outs = [ops.oda_decode_full(qt, hc.kv, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), ws=ws).cpu().numpy()
            for _ in range(2)]
    assert np.array_equal(outs[0], outs[1])
    for b, n in enumerate(ns):
        k, v = hc.k[b].copy(), hc.v[b].copy()
        oracle.oda.commit(k, v, n, kn[b], vn[b])
        keys = keysets.full_keys(n)
        ref = attention.attend(q[b], k, v, keys, SCALE)
        check_tight(outs[0][b], ref, q[b], k, v, keys, SCALE, what="b=%d n=%d" % (b, n))
        kr, vr = ops.kv_read(hc.kv, b, n - 1, 1)
        assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b]) and np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b])
    assert ops.workspace_error(ws) == 0


def test_maximum_batch():
    # 1024 requests (the library's maximum batch), short ragged histories
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    g = np.random.default_rng(64)
    B = 1024
    ns = [int(x) for x in g.integers(1, 48, size=B)]
    hc = HostCache(Hq, Hkv, ns, seed=65, poison=False)
    q = _q(Hq, B, seed=66)
    out = ops.oda_decode_full(torch.as_tensor(q, device="cuda"), hc.kv).cpu().numpy()
    for b in range(0, B, 7):
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.full_keys(ns[b]), SCALE)
        check_tight(out[b], ref, q[b], hc.k[b], hc.v[b], keysets.full_keys(ns[b]), SCALE, what="b=%d" % b)


def test_keep_mask_modes():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    ns = [100, 33000, 5, 1]
    hc = HostCache(Hq, Hkv, ns, seed=40, max_blocks=2100)
    decl = np.array([[gather.FOCUS, 1, 3, 5], [gather.GLOBAL, 0, 0, 0], [gather.LOCAL, 0, 0, 0],
                     [gather.FOCUS, 0, 10, 0]], np.int32)
    m = ops.da_keep_mask(torch.as_tensor(decl, device="cuda"), hc.kv, local_tokens=20).cpu().numpy().view(np.uint32)
    for b, n in enumerate(ns):
        exp = gather.da_mode_blocks(int(decl[b, 0]), n, int(decl[b, 1]), int(decl[b, 2]), int(decl[b, 3]),
                                    local_tokens=20)
        words = np.zeros(m.shape[1], np.uint32)
        for blk in exp:
            words[blk // 32] |= np.uint32(1 << (blk % 32))
        assert np.array_equal(m[b], words), b


def test_recall_head_small():
    from sparse_kv_recall_amd import ops
    g = np.random.default_rng(3)
    for B, din, hid in ((1, 6144, 512), (3, 100, 7), (5, 2048, 33), (64, 512, 128), (2, 20000, 40)):
        x = g.standard_normal((B, din)).astype(np.float32)
        W1 = (g.standard_normal((hid, din)) * 0.02).astype(np.float32)
        b1 = (g.standard_normal(hid) * 0.1).astype(np.float32)
        w2 = (g.standard_normal(hid) * 0.02).astype(np.float32)
        b2 = np.array([0.01], np.float32)
        dev = lambda a: torch.as_tensor(a, device="cuda")
        qo, go = ops.oda_recall_score(dev(x), dev(W1), dev(b1), dev(w2), dev(b2), theta=0.0)
        qo, go = qo.cpu().numpy(), go.cpu().numpy()
        q2, _ = ops.oda_recall_score(dev(x), dev(W1), dev(b1), dev(w2), dev(b2), theta=0.0)
        assert np.array_equal(q2.cpu().numpy(), qo)  # fixed reduction order
        for b in range(B):
            ref = oracle.recall.recall_score(x[b], W1, b1, w2, b2)
            assert abs(qo[b] - ref) <= 1e-5 * max(1.0, abs(ref)), (qo[b], ref)
            if abs(ref) >= 1e-4:
                assert bool(go[b]) == oracle.recall.gate(ref, 0.0)


def test_gate_scores_and_modes():
    from sparse_kv_recall_amd import ops
    s = torch.tensor([0.5, 0.0, -0.0, -1.0, 1e-30, float("nan")], device="cuda")
    out = ops.oda_gate_scores(s, 0.0).cpu().numpy()
    assert out.tolist() == [1, 0, 0, 0, 1, 0]
    fb = torch.tensor([0, 2, 2, 0, 0, 2], dtype=torch.int32, device="cuda")
    out = ops.oda_gate_scores(s, 0.0, fallback=fb).cpu().numpy()
    assert out.tolist() == [1, 2, 2, 0, 1, 2]


def test_invalid_lengths_set_device_error_and_zero_rows():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    hc = HostCache(Hq, Hkv, [50, 60], seed=50)
    hc.set_lens([0, 60])
    ws = ops.workspace(2, Hq)
    q = _q(Hq, 2, seed=13)
    out = torch.full((2, Hq, 128), 3.0, device="cuda")
    ops.oda_decode_full(torch.as_tensor(q, device="cuda"), hc.kv, out=out, ws=ws)
    err = ops.workspace_error(ws)
    assert err & 2
    got = out.cpu().numpy()
    assert (got[0] == 0).all()
    ref = attention.attend(q[1], hc.k[1], hc.v[1], keysets.full_keys(60), SCALE)
    check_tight(got[1], ref, q[1], hc.k[1], hc.v[1], keysets.full_keys(60), SCALE)


def test_kv_write_read_roundtrip_and_layout():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    hc = HostCache(Hq, Hkv, [77], seed=60, permute=True)
    k, v = ops.kv_read(hc.kv, 0, 0, 77)
    assert np.array_equal(bf16_tensor_to_bits(k), hc.k[0][:77])
    assert np.array_equal(bf16_tensor_to_bits(v), hc.v[0][:77])
    # documented tile byte order
    kp = bf16_tensor_to_bits(hc.kv.k_pool).reshape(hc.kv.num_phys_blocks, Hkv, 2048)
    vp = bf16_tensor_to_bits(hc.kv.v_pool).reshape(hc.kv.num_phys_blocks, Hkv, 2048)
    for pos in (0, 5, 16, 40, 76):
        blk, t = pos // 16, pos % 16
        p = hc.bt[0][blk]
        for g in (0, 7):
            for d in (0, 7, 8, 31, 32, 100, 127):
                assert kp[p, g, ((d // 8) * 256 + t * 16 + (d % 8) * 2) // 2] == hc.k[0][pos, g, d]
                off = (d // 32) * 1024 + (t // 4) * 256 + (d % 16) * 16 + ((d // 16) % 2) * 8 + (t % 4) * 2
                assert vp[p, g, off // 2] == hc.v[0][pos, g, d]


def test_deterministic_replay():
    # Split partials cross workgroups and XCDs: a stale read would make repeated launches
    # disagree. Alternate two caches so that each launch starts from different cache state.
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    hcs = [HostCache(Hq, Hkv, [40000, 3000, 131], seed=70 + i, poison=False) for i in range(2)]
    q = torch.as_tensor(_q(Hq, 3, seed=14), device="cuda")
    ws = ops.workspace(3, Hq)
    first = [ops.oda_decode_full(q, hc.kv, ws=ws).cpu().numpy() for hc in hcs]
    for b, n in enumerate([40000, 3000, 131]):
        ref = attention.attend(q.cpu().numpy()[b], hcs[0].k[b], hcs[0].v[b], keysets.full_keys(n), SCALE)
        check_tight(first[0][b], ref, q.cpu().numpy()[b], hcs[0].k[b], hcs[0].v[b], keysets.full_keys(n), SCALE)
    for rep in range(20):
        for i, hc in enumerate(hcs):
            o = ops.oda_decode_full(q, hc.kv, ws=ws)
            o2 = ops.oda_decode_local(q, hc.kv, ws=ws)
            assert np.array_equal(o.cpu().numpy(), first[i]), rep
            assert np.isfinite(o2.cpu().numpy()).all()


@pytest.mark.parametrize("with_sel", [False, True])
def test_kv_append_standalone(with_sel):
    # the stand-alone commit writes the current token into slot n-1 of every selected
    # request and nothing else; an invalid length sets the device error bit
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    ns = [1, 16, 17, 300, 4097, 33]
    hc = HostCache(Hq, Hkv, ns, seed=90)
    B = len(ns)
    kn = rand_bits(rng.mix_key(906, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(906, 2), B, Hkv)
    sel = torch.tensor([1, 0, 1, 1, 0, 1], dtype=torch.int32, device="cuda") if with_sel else None
    ws = ops.workspace(B, Hq)
    ops.kv_append(hc.kv, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), sel=sel, sel_value=1, ws=ws)
    torch.cuda.synchronize()
    assert ops.workspace_error(ws) == 0
    for b, n in enumerate(ns):
        k, v = hc.k[b][:n].copy(), hc.v[b][:n].copy()
        if sel is None or int(sel[b]) == 1:
            oracle.oda.commit(k, v, n, kn[b], vn[b])
        kr, vr = ops.kv_read(hc.kv, b, 0, n)
        assert np.array_equal(bf16_tensor_to_bits(kr), k), b
        assert np.array_equal(bf16_tensor_to_bits(vr), v), b
    # a request of length 0 is refused on the device: error bit, nothing written
    hc.set_lens([0] + ns[1:])
    ws = ops.workspace(B, Hq)
    ops.kv_append(hc.kv, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), ws=ws)
    assert ops.workspace_error(ws) & 2  # SK_DEVERR_SEQ_LEN


@pytest.mark.parametrize("view", ["full", "list"])
def test_single_request_instance_equals_small_batch_plan(view):
    # A launch on one request runs its own kernel instance, whose plan is the small-batch
    # plan for that request alone on the same grid. With at least 256 blocks per request
    # table both launches get the full grid, so the same request in a batch of two, the
    # other request filtered out by the selector, must give the same output bits.
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    for n in (3, 2069, 9000, 40001):
        hc = HostCache(Hq, Hkv, [n, 700], seed=95, max_blocks=2600)
        q = _q(Hq, 2, seed=96)
        qt = torch.as_tensor(q, device="cuda")
        kn = bits_to_bf16_tensor(rand_bits(rng.mix_key(907, 1), 2, Hkv))
        vn = bits_to_bf16_tensor(rand_bits(rng.mix_key(907, 2), 2, Hkv))
        one = ops.PagedKVCache(hc.kv.num_phys_blocks, 1, Hq, Hkv, hc.max_blocks,
                               block_tables=hc.kv.block_tables[:1].contiguous(),
                               seq_lens=hc.kv.seq_lens[:1].contiguous(), k_pool=hc.kv.k_pool, v_pool=hc.kv.v_pool)
        sel = torch.tensor([1, 0], dtype=torch.int32, device="cuda")
        nb = (n + 15) // 16
        kept = sorted(set(range(0, nb, 3)) | {nb - 1})
        mask = torch.as_tensor(_mask_words([kept, [0]], hc.max_blocks).view(np.int32), device="cuda")
        outs = []
        for batch_of_two in (False, True):
            kv = hc.kv if batch_of_two else one
            s = sel if batch_of_two else None
            qq = qt if batch_of_two else qt[:1].contiguous()
            kk = kn if batch_of_two else kn[:1].contiguous()
            vv = vn if batch_of_two else vn[:1].contiguous()
            out = torch.zeros((kv.batch, Hq, 128), device="cuda")
            if view == "full":
                ops.oda_decode_full(qq, kv, kk, vv, sel=s, sel_value=1, out=out)
            else:
                m = mask if batch_of_two else mask[:1].contiguous()
                ops.da_decode_blocks(qq, kv, m, kk, vv, sel=s, sel_value=1, out=out)
            outs.append(out[0].cpu().numpy())
            # restore the slot the commit wrote, so the second launch starts from the same history
            ops.kv_write(hc.kv, 0, n - 1, bits_to_bf16_tensor(hc.k[0][n - 1:n]), bits_to_bf16_tensor(hc.v[0][n - 1:n]))
        assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32)), (view, n)
        keys = keysets.full_keys(n) if view == "full" else keysets.block_keys(n, kept)
        k, v = hc.k[0].copy(), hc.v[0].copy()
        oracle.oda.commit(k, v, n, bf16_tensor_to_bits(kn)[0], bf16_tensor_to_bits(vn)[0])
        ref = attention.attend(q[0], k, v, keys, SCALE)
        check_tight(outs[0], ref, q[0], k, v, keys, SCALE, what="%s n=%d" % (view, n))


def test_single_request_local_view_commit_tile_alone():
    # At one request the Local view's last split can hold only the tile that receives the
    # current token, which its wave then takes from its first request: lengths that put 0,
    # 1 and 2 window positions in the last block, with the commit checked bit for bit
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    for n in (2069, 2070, 2084, 4097, 4112):
        hc = HostCache(Hq, Hkv, [n], seed=97)
        q = _q(Hq, 1, seed=98)
        kn = rand_bits(rng.mix_key(908, n, 1), 1, Hkv)
        vn = rand_bits(rng.mix_key(908, n, 2), 1, Hkv)
        out = ops.oda_decode_local(torch.as_tensor(q, device="cuda"), hc.kv, bits_to_bf16_tensor(kn),
                                   bits_to_bf16_tensor(vn)).cpu().numpy()
        k, v = hc.k[0].copy(), hc.v[0].copy()
        oracle.oda.commit(k, v, n, kn[0], vn[0])
        keys = keysets.local_keys(n)
        ref = attention.attend(q[0], k, v, keys, SCALE)
        check_tight(out[0], ref, q[0], k, v, keys, SCALE, what="local n=%d" % n)
        kr, vr = ops.kv_read(hc.kv, 0, n - 1, 1)
        assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[0]) and np.array_equal(bf16_tensor_to_bits(vr)[0], vn[0])


def test_single_request_invalid_length_and_empty_list():
    # the single-request instance's own handling of a request it cannot attend: a length of
    # 0 or past the block table sets SK_DEVERR_SEQ_LEN and zeroes the row; an empty
    # gathered list sets SK_DEVERR_EMPTY, zeroes the row and still commits the token
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    hc = HostCache(Hq, Hkv, [300], seed=99)
    q = torch.as_tensor(_q(Hq, 1, seed=100), device="cuda")
    for bad_n in (0, hc.max_blocks * 16 + 1):
        hc.set_lens([bad_n])
        for call in ("full", "local"):
            ws = ops.workspace(1, Hq)
            out = torch.full((1, Hq, 128), 5.0, device="cuda")
            if call == "full":
                ops.oda_decode_full(q, hc.kv, out=out, ws=ws)
            else:
                ops.oda_decode_local(q, hc.kv, out=out, ws=ws)
            assert ops.workspace_error(ws) & 2, (bad_n, call)
            assert not out.cpu().numpy().any(), (bad_n, call)
    hc.set_lens([300])
    kn = rand_bits(rng.mix_key(909, 1), 1, Hkv)
    vn = rand_bits(rng.mix_key(909, 2), 1, Hkv)
    gat = torch.zeros((1, hc.max_blocks), dtype=torch.int32, device="cuda")
    cnt = torch.zeros_like(gat)
    num = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = ops.workspace(1, Hq)
    out = torch.full((1, Hq, 128), 5.0, device="cuda")
    ops.da_decode_gathered(q, hc.kv, gat, cnt, num, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), out=out, ws=ws)
    assert ops.workspace_error(ws) & 4  # SK_DEVERR_EMPTY
    assert not out.cpu().numpy().any()
    kr, vr = ops.kv_read(hc.kv, 0, 299, 1)
    assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[0]) and np.array_equal(bf16_tensor_to_bits(vr)[0], vn[0])


@pytest.mark.parametrize("Hq,Hkv", [(12, 3), (10, 5), (16, 16), (48, 3)])
def test_odd_and_wide_kv_head_counts(Hq, Hkv):
    # The split plan gives each KV head grid / Hkv slots; with 3, 5 or 16 KV heads the grid
    # (a multiple of 8 workgroups) does not divide evenly. Batch instance (four ragged
    # requests): Full, Local and a block list; single-request instance: Full with the
    # current token committed, Local with and without the step's tile table, a block list.
    from sparse_kv_recall_amd import ops
    g = np.random.default_rng(Hq * 100 + Hkv)
    ns = [37, 4500, 2100, 9000]
    hc = HostCache(Hq, Hkv, ns, seed=Hq * 10 + Hkv)
    q = _q(Hq, len(ns), seed=Hq + 7 * Hkv)
    qt = torch.as_tensor(q, device="cuda")
    kept = []
    for n in ns:
        nb = (n + 15) // 16
        kept.append(sorted(set(g.choice(nb, size=max(1, nb // 8), replace=False).tolist()) | {nb - 1}))
    mask = torch.as_tensor(_mask_words(kept, hc.max_blocks).view(np.int32), device="cuda")
    ws = ops.workspace(len(ns), Hq)
    outs = {"full": ops.oda_decode_full(qt, hc.kv, ws=ws).cpu().numpy(),
            "local": ops.oda_decode_local(qt, hc.kv, ws=ws).cpu().numpy(),
            "list": ops.da_decode_blocks(qt, hc.kv, mask, ws=ws)[0].cpu().numpy()}
    assert ops.workspace_error(ws) == 0
    for b, n in enumerate(ns):
        for view, keys in (("full", keysets.full_keys(n)), ("local", keysets.local_keys(n)),
                           ("list", keysets.block_keys(n, kept[b]))):
            ref = attention.attend(q[b], hc.k[b], hc.v[b], keys, SCALE)
            check_tight(outs[view][b], ref, q[b], hc.k[b], hc.v[b], keys, SCALE,
                        what="batch %s Hq=%d Hkv=%d n=%d" % (view, Hq, Hkv, n))

    n = 9000
    one = HostCache(Hq, Hkv, [n], seed=Hq * 10 + Hkv + 1)
    q1 = _q(Hq, 1, seed=Hq + 7 * Hkv + 1)
    q1t = torch.as_tensor(q1, device="cuda")
    kn = rand_bits(rng.mix_key(902, Hq, Hkv, 1), 1, Hkv)
    vn = rand_bits(rng.mix_key(902, Hq, Hkv, 2), 1, Hkv)
    ws1 = ops.workspace(1, Hq)
    loc = ops.oda_decode_local(q1t, one.kv, ws=ws1).cpu().numpy()
    tab = ops.local_tiles(one.kv)
    loc_tab = ops.oda_decode_local_tiles(q1t, one.kv, tab, ws=ws1).cpu().numpy()
    assert np.array_equal(loc.view(np.uint32), loc_tab.view(np.uint32)), "tile table changed the Local view"
    nb = (n + 15) // 16
    kept1 = sorted(set(g.choice(nb, size=nb // 8, replace=False).tolist()) | {nb - 1})
    mask1 = torch.as_tensor(_mask_words([kept1], one.max_blocks).view(np.int32), device="cuda")
    lst = ops.da_decode_blocks(q1t, one.kv, mask1, ws=ws1)[0].cpu().numpy()
    full = ops.oda_decode_full(q1t, one.kv, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), ws=ws1).cpu().numpy()
    k_got, v_got = ops.kv_read(one.kv, 0, n - 1, 1)
    assert np.array_equal(bf16_tensor_to_bits(k_got)[0], kn[0]) and np.array_equal(bf16_tensor_to_bits(v_got)[0],
                                                                                   vn[0])
    kb, vb = one.k[0].copy(), one.v[0].copy()
    kb[n - 1], vb[n - 1] = kn[0], vn[0]
    for view, got, keys, kk, vv in (("local", loc, keysets.local_keys(n), one.k[0], one.v[0]),
                                    ("list", lst, keysets.block_keys(n, kept1), one.k[0], one.v[0]),
                                    ("full+commit", full, keysets.full_keys(n), kb, vb)):
        ref = attention.attend(q1[0], kk, vv, keys, SCALE)
        check_tight(got[0], ref, q1[0], kk, vv, keys, SCALE, what="single %s Hq=%d Hkv=%d" % (view, Hq, Hkv))
    assert ops.workspace_error(ws1) == 0
