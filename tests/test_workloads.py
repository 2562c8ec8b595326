"""The synthetic workloads have the shapes and statistics their recipe states."""
import numpy as np

import moe_workloads as W


def test_tiny_and_qwen3_shapes():
    t = W.tiny()
    assert t.x.shape == (64, 256) and t.ids.shape == (64, 2) and t.probs.dtype == np.float32
    assert np.allclose(t.probs.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(t.probs, axis=1) <= 0)  # slots in descending probability
    assert all(len(set(r)) == 2 for r in t.ids.tolist())
    q = W.qwen3(T=4096)
    c = q.expert_counts()
    assert c.sum() == 4096 * 8 and c.min() > 150 and c.max() < 400  # near-uniform load
    assert q.w1(0).shape == (1536, 2048) and q.w2(127).shape == (2048, 768)
    w = W.bf16_bits_to_f32(q.w1(3)).astype(np.float64)
    assert abs(w.std() - 0.02) < 1e-3


def test_skewed_routing_follows_zipf():
    s = W.skewed(T=16384)
    c = s.expert_counts()
    assert c.max() > 2000 and (c <= 8).sum() >= 1 and c.sum() == 16384 * 8


def test_dense_outliers():
    d = W.dense()
    assert d.n_outliers == 83886
    x = np.abs(W.bf16_bits_to_f32(d.x))
    assert (x > 10).sum() > 0.5 * d.n_outliers


def test_generators_are_seeded():
    a, b = W.tiny(seed=0), W.tiny(seed=0)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w1(3), b.w1(3))
    assert not np.array_equal(W.tiny(seed=1).x, a.x)
