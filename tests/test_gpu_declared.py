"""GPU parity of da_decode_declared, the declared-mode view whose block-table rewrite runs
inside the decode kernel: against the fp64 oracle (the mode's kept blocks, then attention
over their positions) and bit for bit against the keep mask + gathered list path
(da_keep_mask, then da_decode_blocks), which attends the same tiles in the same order.
Declarations cover every mode and the edge cases of the focus interval (empty, reversed,
negative, past the end, overlapping or adjacent to the output blocks, nothing kept)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import attention, gather, keysets
from synth import rng
from tests.helpers import (SCALE, HostCache, bf16_tensor_to_bits, bits_to_bf16_tensor, check_close, check_tight,
                           rand_bits, rand_f32, requires_gpu)

pytestmark = [pytest.mark.gpu, requires_gpu]

G_, F_, L_ = gather.GLOBAL, gather.FOCUS, gather.LOCAL
# (n, decl)
CASES = [
    (1, (G_, 0, 0, 0)),
    (4097, (G_, 0, 0, 0)),
    (100, (F_, 1, 3, 5)),              # focus run + output run
    (300, (F_, 9, 4, 2)),              # reversed focus interval: only the output blocks
    (2000, (F_, 10, 100, 5)),          # output run starts before the focus run: one run
    (500, (F_, 2, 6, 6)),              # adjacent runs: one run
    (600, (F_, -5, 3, 1000)),          # negative begin, output past the end: [0, 3) only
    (700, (F_, 30, 5000, 40)),         # focus past the end, overlapping the output run
    (320, (F_, 5, 5, 100)),            # nothing kept: empty key set
    (33, (F_, 0, 1, 3)),               # focus [0, 1), output past the end: token not attended
    (33000, (L_, 0, 0, 0)),
    (5, (L_, 0, 0, 0)),
    (2048, (7, 0, 0, 0)),              # not a mode: nothing kept
]


def _expected_blocks(n, d, local_tokens):
    if d[0] not in (G_, F_, L_):
        return []
    return gather.da_mode_blocks(d[0], n, d[1], d[2], d[3], local_tokens=local_tokens)


def _mask_of(blocks_per_req, max_blocks):
    words = np.zeros((len(blocks_per_req), (max_blocks + 31) // 32), np.uint32)
    for b, kept in enumerate(blocks_per_req):
        for blk in kept:
            words[b, blk // 32] |= np.uint32(1 << (blk % 32))
    return words


@pytest.mark.parametrize("local_tokens", [0, 20, 1024])
@pytest.mark.parametrize("commit", [False, True])
def test_declared_matches_oracle_and_list_path(local_tokens, commit):
    _declared_case(local_tokens, commit, 32, 8)


@pytest.mark.parametrize("Hq,Hkv", [(15, 3), (16, 16)])
def test_declared_odd_and_wide_kv_head_counts(Hq, Hkv):
    # split slots per KV head that leave a remainder of the grid (3 KV heads), one q head per
    # KV head (16)
    _declared_case(1024, True, Hq, Hkv)


def _declared_case(local_tokens, commit, Hq, Hkv):
    from sparse_kv_recall_amd import ops
    ns = [n for n, _ in CASES]
    decl = np.array([d for _, d in CASES], np.int32)
    B = len(ns)
    hc_d = HostCache(Hq, Hkv, ns, seed=70, max_blocks=2100)  # declared path
    hc_l = HostCache(Hq, Hkv, ns, seed=70, max_blocks=2100)  # keep mask + list path (same contents)
    q = rand_f32(rng.mix_key(970, local_tokens), (B, Hq, 128), 1.0)
    qt = torch.as_tensor(q, device="cuda")
    kn = rand_bits(rng.mix_key(971, 1), B, Hkv)
    vn = rand_bits(rng.mix_key(971, 2), B, Hkv)
    kw = dict(k_new=bits_to_bf16_tensor(kn), v_new=bits_to_bf16_tensor(vn)) if commit else {}
    dt = torch.as_tensor(decl, device="cuda")
    ws_d = ops.workspace(B, Hq)
    ws_l = ops.workspace(B, Hq)
    out_d = ops.da_decode_declared(qt, hc_d.kv, dt, local_tokens=local_tokens, ws=ws_d, **kw)
    mask = ops.da_keep_mask(dt, hc_l.kv, local_tokens=local_tokens)
    out_l, _, _, _ = ops.da_decode_blocks(qt, hc_l.kv, mask, ws=ws_l, **kw)
    torch.cuda.synchronize()
    got, ref_l = out_d.cpu().numpy(), out_l.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref_l.view(np.uint32))
    assert ops.workspace_error(ws_d) == ops.workspace_error(ws_l) == 4  # SK_DEVERR_EMPTY (two empty sets)
    for b, n in enumerate(ns):
        kept = _expected_blocks(n, decl[b], local_tokens)
        k, v = hc_d.k[b].copy(), hc_d.v[b].copy()
        if commit:
            oracle.oda.commit(k, v, n, kn[b], vn[b])
            kr, vr = ops.kv_read(hc_d.kv, b, n - 1, 1)
            assert np.array_equal(bf16_tensor_to_bits(kr)[0], kn[b]), b
            assert np.array_equal(bf16_tensor_to_bits(vr)[0], vn[b]), b
        if not kept:
            assert not got[b].any(), b  # empty key set: zero row
            continue
        ref = attention.attend(q[b], k, v, keysets.block_keys(n, kept), SCALE)
        check_tight(got[b], ref, q[b], k, v, keysets.block_keys(n, kept), SCALE,
                    what="declared n=%d decl=%s" % (n, decl[b]))


def test_declared_with_selector_skips_requests():
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 16, 4
    ns = [3000, 70, 12000]
    decl = np.array([[F_, 3, 40, 180], [G_, 0, 0, 0], [L_, 0, 0, 0]], np.int32)
    hc = HostCache(Hq, Hkv, ns, seed=72)
    q = rand_f32(rng.mix_key(972), (3, Hq, 128), 1.0)
    out = torch.full((3, Hq, 128), 7.0, device="cuda")
    sel = torch.tensor([2, 1, 2], dtype=torch.int32, device="cuda")
    ops.da_decode_declared(torch.as_tensor(q, device="cuda"), hc.kv, torch.as_tensor(decl, device="cuda"),
                           local_tokens=1024, sel=sel, sel_value=2, out=out)
    got = out.cpu().numpy()
    assert (got[1] == 7.0).all()  # not selected: untouched
    for b in (0, 2):
        kept = gather.da_mode_blocks(int(decl[b, 0]), ns[b], int(decl[b, 1]), int(decl[b, 2]), int(decl[b, 3]),
                                     local_tokens=1024)
        ref = attention.attend(q[b], hc.k[b], hc.v[b], keysets.block_keys(ns[b], kept), SCALE)
        check_tight(got[b], ref, q[b], hc.k[b], hc.v[b], keysets.block_keys(ns[b], kept), SCALE)


def test_declared_large_batch_matches_list_path():
    """Batches above 64 take the workgroup (LDS) planning path: 100 ragged requests with
    seeded declarations of every mode, bit for bit against mask + list, with commits."""
    from sparse_kv_recall_amd import ops
    Hq, Hkv = 8, 2
    g = np.random.default_rng(73)
    B = 100
    ns = [int(x) for x in g.integers(1, 3000, size=B)]
    ns[:3] = [1, 16, 2999]
    decl = np.zeros((B, 4), np.int32)
    for b, n in enumerate(ns):
        nb = (n + 15) // 16
        mode = int(g.integers(0, 3))
        fb = int(g.integers(-2, nb + 2))
        decl[b] = (mode, fb, fb + int(g.integers(0, 40)), int(g.integers(0, nb + 3)))
    hc_d = HostCache(Hq, Hkv, ns, seed=74)
    hc_l = HostCache(Hq, Hkv, ns, seed=74)
    q = torch.as_tensor(rand_f32(rng.mix_key(974), (B, Hq, 128), 1.0), device="cuda")
    kn = bits_to_bf16_tensor(rand_bits(rng.mix_key(975, 1), B, Hkv))
    vn = bits_to_bf16_tensor(rand_bits(rng.mix_key(975, 2), B, Hkv))
    dt = torch.as_tensor(decl, device="cuda")
    out_d = ops.da_decode_declared(q, hc_d.kv, dt, local_tokens=300, k_new=kn, v_new=vn)
    mask = ops.da_keep_mask(dt, hc_l.kv, local_tokens=300)
    out_l, _, _, _ = ops.da_decode_blocks(q, hc_l.kv, mask, k_new=kn, v_new=vn)
    torch.cuda.synchronize()
    assert np.array_equal(out_d.cpu().numpy().view(np.uint32), out_l.cpu().numpy().view(np.uint32))
    for b, n in enumerate(ns):
        kd, vd = ops.kv_read(hc_d.kv, b, 0, n)
        kl, vl = ops.kv_read(hc_l.kv, b, 0, n)
        assert np.array_equal(bf16_tensor_to_bits(kd), bf16_tensor_to_bits(kl)), b
        assert np.array_equal(bf16_tensor_to_bits(vd), bf16_tensor_to_bits(vl)), b
