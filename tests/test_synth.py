"""CPU checks of the synthetic input generators (no method arithmetic here)."""

import math

import numpy as np
import torch

from synth import rng, workloads


def test_splitmix_vectorised_matches_scalar_definition():
    for key in (0, 1, rng.mix_key(3, 4, 5), (1 << 64) - 1):
        ref = [rng.splitmix64_scalar(key, i) for i in range(1000, 1100)]
        got = rng._raw(key, 1000, 100)
        assert [int(x) for x in got] == ref


def test_splitmix_known_sequence():
    # SplitMix64 with seed 0 starts 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F
    assert [rng.splitmix64_scalar(0, i) for i in range(3)] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                                               0x06C45D188009454F]


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32) * 3,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(rng.f32_to_bf16_bits(x), ref)


def test_normal_stream_moments_and_slicing():
    key = rng.mix_key(7, 7)
    x = rng.normal_f32(key, 0, 1 << 21, rng.unit_scale()).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    assert np.abs(x).max() <= 2 * math.sqrt(3) + 1e-6
    # any slice equals the same slice of the whole stream (threaded chunks included)
    y = rng.normal_f32(key, 12345, 5 * (1 << 22) + 17, rng.unit_scale())
    z = rng.normal_f32(key, 12345 + 4 * (1 << 22), (1 << 22) + 17, rng.unit_scale())
    assert np.array_equal(y[4 * (1 << 22):], z)
    w = rng.normal_f32(key, 100, 50, rng.unit_scale(0.02))
    assert np.array_equal(w, (x[100:150].astype(np.float32) / rng.unit_scale() * 0 + w))


def test_scaled_stream_is_one_rounding():
    key = rng.mix_key(8, 8)
    z = rng._raw(key, 0, 1000)
    m = np.uint64(0xFFFF)
    c = ((z & m).astype(np.int64) + ((z >> np.uint64(16)) & m).astype(np.int64) +
         ((z >> np.uint64(32)) & m).astype(np.int64) + (z >> np.uint64(48)).astype(np.int64) - 131070)
    s = rng.unit_scale(0.02)
    exp = (c.astype(np.float64) * np.float64(s)).astype(np.float32)  # exact product rounded once
    assert np.array_equal(rng.normal_f32(key, 0, 1000, s), exp)


def test_workload_invariants():
    w1 = workloads.oda_small()
    assert w1.steps == 64 and w1.Hq == 8 and w1.Hkv == 2
    w3 = workloads.oda_stack128k()
    assert int((w3.sched_scores > 0).sum()) == 128
    # one recall in every aligned run of 8 steps, at offsets that are not all the same
    runs = (w3.sched_scores[:, 0] > 0).reshape(128, 8)
    assert (runs.sum(axis=1) == 1).all()
    assert len(set(np.argmax(runs, axis=1).tolist())) > 4
    assert w3.n_at(0)[0] == 131073 and w3.n_at(1023)[0] == 132096
    w4 = workloads.da_32k()
    assert sorted(w4.block_tables[0].tolist()) == list(range(w4.num_phys_blocks))
    assert w4.num_phys_blocks == 2080
    modes = w4.decl[:, 0, 0]
    assert set(modes.tolist()) == {0, 1, 2}
    foc = w4.decl[modes == workloads.DA_FOCUS, 0]
    assert (foc[:, 2] - foc[:, 1] == 128).all() and (foc[:, 1] >= 0).all() and (foc[:, 2] <= 1984).all()
    w5 = workloads.ragged32()
    assert w5.H0.min() >= 4096 and w5.H0.max() <= 131072
    used = w5.block_tables[w5.block_tables >= 0]
    assert sorted(used.tolist()) == list(range(w5.num_phys_blocks))
    for r in range(w5.batch):
        existing = (int(w5.H0[r]) + 15) // 16
        bits = [(int(w5.keep_mask[r, b // 32]) >> (b % 32)) & 1 for b in range(existing)]
        first_new = int(w5.H0[r]) // 16
        kept_old = sum(bits[:first_new])
        f = w5.extra["keep_fraction"][r]
        assert 0.05 <= f <= 0.20
        assert abs(kept_old - f * existing) <= 2 + 1
        assert all(bits[first_new:])
    assert set(w5.fallback.tolist()) <= {workloads.MODE_LOCAL, workloads.MODE_BLOCKS}


def test_candidates_layer0_share_passes():
    w = workloads.oda_stack16k(layers=3)
    assert np.array_equal(w.cand_q(5, 0, 0, 0), w.cand_q(5, 0, 1, 0))
    assert not np.array_equal(w.cand_q(5, 1, 0, 0), w.cand_q(5, 1, 1, 0))
    k0, v0 = w.cand_kv(5, 0, 0, 0)
    k1, v1 = w.cand_kv(5, 0, 1, 0)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)


def test_decoder_workload_is_deterministic():
    from synth.decoder import decoder_small
    a, b = decoder_small(), decoder_small()
    wa, wb = a.host_weights(), b.host_weights()
    assert set(wa) == set(wb)
    for k in wa:
        assert np.array_equal(wa[k], wb[k]), k
    assert wa["qkv.0"].shape == ((4 + 2 * 2) * 128, 512) and wa["qkv.0"].dtype == np.uint16
    assert wa["W1"].dtype == np.float32 and wa["W1"].shape == (64, 3 * 512)
    assert np.array_equal(a.tokens, b.tokens) and a.tokens.max() < a.vocab
