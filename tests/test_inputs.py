"""Seeded input generator: determinism, storage rounding and value laws."""

import numpy as np
import torch

import ssm_inputs as gen


def test_same_seed_same_bytes():
    a = gen.make_scan(2, 9, 7, 4, dtype="bf16", seed=5)
    b = gen.make_scan(2, 9, 7, 4, dtype="bf16", seed=5)
    for name in ("x", "delta", "z", "Bm", "Cm"):
        np.testing.assert_array_equal(getattr(a, name).bf16, getattr(b, name).bf16)
    np.testing.assert_array_equal(a.A, b.A)
    np.testing.assert_array_equal(a.h0, b.h0)


def test_streams_do_not_shift():
    """Turning the gate off must not change any other tensor."""
    a = gen.make_scan(2, 9, 7, 4, dtype="f32", seed=6, gate=True)
    b = gen.make_scan(2, 9, 7, 4, dtype="f32", seed=6, gate=False)
    np.testing.assert_array_equal(a.x.f32, b.x.f32)
    np.testing.assert_array_equal(a.Cm.f32, b.Cm.f32)
    np.testing.assert_array_equal(a.h0, b.h0)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    ours = gen.bf16_round(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_to_f32(ours), torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_value_laws():
    w = gen.make_scan(1, 512, 64, 16, dtype="f32", seed=1)
    assert (w.delta.f32 > 0).all()
    assert (w.A <= -1.0 + 1e-6).all() and (w.A >= -16.0 - 1e-4).all()
    assert abs(float(np.std(w.h0)) - 0.5) < 0.05
    assert abs(float(np.std(w.x.f32)) - 1.0) < 0.05
    sp = np.log1p(np.exp(-1.0))
    assert abs(float(np.median(w.delta.f32)) - sp) < 0.02


def test_workload_shapes():
    s = gen.make_workload("tiny_fp32")
    assert s.x.shape == (1, 64, 16) and s.A.shape == (16, 4) and s.h0.shape == (1, 16, 4)
    d = gen.make_decode(3, 8, 16, 5)
    assert d.x.shape == (5, 3, 8) and d.Bm.shape == (5, 3, 16) and d.state0.shape == (3, 8, 16)
    q = gen.make_ssd(1, 16, 4, 2, 2, 8, chunk=8)
    assert q.x.shape == (1, 16, 4, 2) and q.dt.shape == (1, 16, 4) and q.Bm.shape == (1, 16, 2, 8)


def test_pool_decode_slots_distinct_and_in_range():
    p = gen.make_pool_decode(6, 3, 8, 4, 10, seed=5)
    assert p.tokens.x.shape == (6, 3, 8) and p.tokens.h0 is None and p.pool.shape == (10, 8, 4)
    assert p.slots.dtype == np.int32 and len(set(p.slots.tolist())) == 6
    assert p.slots.min() >= 0 and p.slots.max() < 10
    q = gen.make_pool_decode(6, 3, 8, 4, 10, seed=5)
    assert np.array_equal(p.slots, q.slots) and np.array_equal(p.pool, q.pool)
