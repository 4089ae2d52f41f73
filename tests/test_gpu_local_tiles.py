"""GPU tests of the Local view's tile table (oda_local_tiles) and of the Local view read
through it (oda_decode_local_tiles): the table's blocks against the Local key set of the
pages' definition (sinks, then the window, as disjoint position ranges), and the decode bit
for bit against oda_decode_local, which attends the same tiles in the same order."""

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, keysets
from synth import rng
from tests.helpers import (SCALE, HostCache, bf16_tensor_to_bits, bits_to_bf16_tensor, check_tight, rand_bits,
                           rand_f32, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _single(hc, b):
    """Request b of a HostCache as a one-request cache (the single-request kernel instance)."""
    from sparse_kv_recall_amd import ops
    return ops.PagedKVCache(hc.kv.num_phys_blocks, 1, hc.Hq, hc.Hkv, hc.max_blocks,
                            block_tables=hc.kv.block_tables[b:b + 1].contiguous(),
                            seq_lens=hc.kv.seq_lens[b:b + 1].contiguous(), k_pool=hc.kv.k_pool, v_pool=hc.kv.v_pool)


def _expected_tiles(bt_row, n, sinks, window):
    # the Local key set split into its two ranges, each range's blocks in ascending order
    keys = np.asarray(keysets.local_keys(n, sinks, window))
    s_end = min(sinks, n)
    blocks = [sorted(set(int(j) // 16 for j in keys[keys < s_end])),
              sorted(set(int(j) // 16 for j in keys[keys >= s_end]))]
    return np.asarray([bt_row[blk] for run in blocks for blk in run], np.int32)


@pytest.mark.parametrize("sinks,window", [(4, 2048), (0, 17), (20, 5), (3, 20)])
def test_table_lists_the_local_blocks(sinks, window):
    from sparse_kv_recall_amd import ops
    ns = [1, 3, 4, 5, 17, 25, 2052, 2053, 2069, 4097]
    hc = HostCache(8, 2, ns, seed=sinks * 7 + window, poison=False)
    tab = ops.local_tiles(hc.kv, sinks, window)
    row = ops.local_tiles_bytes(1, sinks, window, hc.max_blocks) // 4
    t = tab.cpu().numpy().reshape(len(ns), row)
    for b, n in enumerate(ns):
        exp = _expected_tiles(hc.bt[b], n, sinks, window)
        assert list(t[b, :3]) == [n, sinks, window]
        assert len(exp) <= row - 3
        assert np.array_equal(t[b, 3:3 + len(exp)], exp), (b, n)


def _run_pair(hc, b, q, kn, vn, sinks, window, tab=None, sel=None, sel_value=0):
    """Request b through oda_decode_local and through oda_decode_local_tiles (with `tab`, or
    a table built now): both outputs; the slot n-1 is restored after each launch."""
    from sparse_kv_recall_amd import ops
    one = _single(hc, b)
    n = hc.ns[b]
    if tab is None:
        tab = ops.local_tiles(one, sinks, window)
    outs = []
    for with_table in (False, True):
        ws = ops.workspace(1, hc.Hq)
        out = torch.full((1, hc.Hq, 128), 7.0, device="cuda")
        args = dict(sinks=sinks, window=window, sel=sel, sel_value=sel_value, out=out, ws=ws)
        if with_table:
            ops.oda_decode_local_tiles(q, one, tab, kn, vn, **args)
        else:
            ops.oda_decode_local(q, one, kn, vn, **args)
        assert ops.workspace_error(ws) == 0
        outs.append(out.cpu().numpy()[0])
        if kn is not None and n >= 1:
            kr, vr = ops.kv_read(one, 0, n - 1, 1)
            outs.append((bf16_tensor_to_bits(kr)[0], bf16_tensor_to_bits(vr)[0]))
            ops.kv_write(one, 0, n - 1, bits_to_bf16_tensor(hc.k[b][n - 1:n]), bits_to_bf16_tensor(hc.v[b][n - 1:n]))
    return outs


@pytest.mark.parametrize("sinks,window", [(4, 2048), (0, 17), (20, 5)])
def test_decode_with_table_equals_without(sinks, window):
    # the single-request instance that reads the table against the one that reads the block
    # table: outputs and committed slots bit for bit, and the oracle's attention
    Hq, Hkv = 32, 8
    ns = [1, 5, 17, 2052, 2053, 2069, 4097, 9000]
    hc = HostCache(Hq, Hkv, ns, seed=sinks + window)
    for b, n in enumerate(ns):
        q = torch.as_tensor(rand_f32(rng.mix_key(940, b), (1, Hq, 128)), device="cuda")
        kn = rand_bits(rng.mix_key(941, b, 1), 1, Hkv)
        vn = rand_bits(rng.mix_key(941, b, 2), 1, Hkv)
        o0, c0, o1, c1 = _run_pair(hc, b, q, bits_to_bf16_tensor(kn), bits_to_bf16_tensor(vn), sinks, window)
        assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), n
        assert np.array_equal(c0[0], kn[0]) and np.array_equal(c0[1], vn[0])
        assert np.array_equal(c1[0], kn[0]) and np.array_equal(c1[1], vn[0])
        k, v = hc.k[b].copy(), hc.v[b].copy()
        oracle.oda.commit(k, v, n, kn[0], vn[0])
        keys = keysets.local_keys(n, sinks, window)
        check_tight(o1, attention.attend(q.cpu().numpy()[0], k, v, keys, SCALE), q.cpu().numpy()[0], k, v, keys,
                    SCALE, what="local via table n=%d s=%d w=%d" % (n, sinks, window))


def test_table_of_another_step_falls_back():
    # a table built at n, used at n + 1 (the window moved by one position, and at n = 2064
    # into a new block), a table built for another window, and a table never built: the
    # launch reads the block table and gives the same bits as without a table
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    ns = [2064, 3000, 40]
    hc = HostCache(Hq, Hkv, [n + 1 for n in ns], seed=950)
    for b, n in enumerate(ns):
        q = torch.as_tensor(rand_f32(rng.mix_key(951, b), (1, Hq, 128)), device="cuda")
        one = _single(hc, b)
        one.seq_lens.fill_(n)
        stale = ops.local_tiles(one, 4, 2048)
        one.seq_lens.fill_(n + 1)
        hc.ns[b] = n + 1
        other_window = ops.local_tiles(one, 4, 2032, tab=torch.zeros_like(stale))
        for tab in (stale, other_window, torch.zeros_like(stale)):
            o0, o1 = _run_pair(hc, b, q, None, None, 4, 2048, tab=tab)
            assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), (n, tab[:3].tolist())


def test_table_with_selector_and_batches():
    # a selector that skips the request writes nothing through either path; a batch of three
    # (the batch instance, which does not read the table) gives the bits of oda_decode_local
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 16, 4
    ns = [2100, 77, 5000]
    hc = HostCache(Hq, Hkv, ns, seed=960)
    q = torch.as_tensor(rand_f32(rng.mix_key(961), (3, Hq, 128)), device="cuda")
    sel = torch.tensor([3], dtype=torch.int32, device="cuda")
    o0, o1 = _run_pair(hc, 0, q[:1].contiguous(), None, None, 4, 2048, sel=sel, sel_value=2)
    assert (o0 == 7.0).all() and (o1 == 7.0).all()
    o0, o1 = _run_pair(hc, 0, q[:1].contiguous(), None, None, 4, 2048, sel=sel, sel_value=3)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)) and not (o0 == 7.0).all()
    tab = ops.local_tiles(hc.kv, 4, 2048)
    a = ops.oda_decode_local(q, hc.kv).cpu().numpy()
    b = ops.oda_decode_local_tiles(q, hc.kv, tab).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_table_entry_outside_the_pool_sets_the_block_error():
    # the table's blocks are checked as the block table's are: an entry outside the pool
    # sets SK_DEVERR_BLOCK_ID (and that tile attends nothing)
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 32, 8
    hc = HostCache(Hq, Hkv, [3000], seed=970)
    one = _single(hc, 0)
    tab = ops.local_tiles(one, 4, 2048)
    tab[7] = hc.kv.num_phys_blocks + 9
    ws = ops.workspace(1, Hq)
    q = torch.as_tensor(rand_f32(rng.mix_key(971), (1, Hq, 128)), device="cuda")
    ops.oda_decode_local_tiles(q, one, tab, ws=ws)
    assert ops.workspace_error(ws) & 1
