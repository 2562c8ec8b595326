"""Pins of the oracle's router (scores and deterministic top-k) to values fixed
independently of it: hand-computed cases, brute-force ranking by Python's own
sort, closed forms of the softmax, and the workload generator's router (a
different formulation: a stable sort of FP64 softmax probabilities).

Sources: the article "Finish RL training faster: bitwise consistent,
high-performance, agent-driven", section 2 (the same discrete choice needs the
same tie-breaking and output order) and section 4.4 ("R3 unnecessary": one
FP32-output scoring kernel for every batch size)."""
import math

import numpy as np
import pytest

import moe_workloads as W
import oracle


def _bf16(a):
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def test_router_logits_hand_example():
    x = _bf16([[1.0, 2.0], [-0.5, 0.25]])
    w = _bf16([[1.0, 1.0], [0.5, -1.0], [0.0, 4.0]])
    got = oracle.router_logits(x, w)
    want = np.array([[3.0, -1.5, 8.0], [-0.25, -0.5, 1.0]])
    assert np.array_equal(got, want)


def test_router_logits_one_hot_picks_a_weight_column():
    rng = np.random.default_rng(11)
    w = _bf16(rng.standard_normal((16, 64)))
    x = np.zeros((64, 64), np.uint16)
    x[np.arange(64), np.arange(64)] = _bf16([1.0])[0]
    got = oracle.router_logits(x, w)
    assert np.array_equal(got, W.bf16_bits_to_f32(w).astype(np.float64).T)
    # scaling x by a power of two scales every score exactly
    x2 = _bf16(W.bf16_bits_to_f32(x) * 8.0)
    assert np.array_equal(oracle.router_logits(x2, w), got * 8.0)


def test_topk_ties_go_to_the_lower_expert_id():
    l = np.array([[1, 3, 3, 2], [0, 0, 0, 0], [5, -1, 5, 5]], np.float32)
    ids, p = oracle.router_topk(l, 2)
    assert ids.tolist() == [[1, 2], [0, 1], [0, 2]]
    assert np.array_equal(p, np.full((3, 2), 0.5, np.float32))
    ids, p = oracle.router_topk(l, 3, renormalize=False)
    assert ids.tolist() == [[1, 2, 3], [0, 1, 2], [0, 2, 3]]
    assert np.allclose(p[1], 0.25) and np.allclose(p[2], 1 / (3 + math.exp(-6)))
    # signed zeros are equal scores
    ids, _ = oracle.router_topk(np.array([[-0.0, 0.0, -1.0]], np.float32), 2)
    assert ids.tolist() == [[0, 1]]


def test_topk_softmax_closed_forms():
    # scores differing by ln 3: renormalized probabilities 3/4 and 1/4
    l = np.array([[math.log(3.0), 0.0, -30.0]], np.float32)
    ids, p = oracle.router_topk(l, 2)
    d = float(l[0, 0]) - float(l[0, 1])
    assert ids.tolist() == [[0, 1]]
    assert p[0, 0] == np.float32(math.exp(d) / (math.exp(d) + 1.0))
    assert abs(p[0, 0] - 0.75) < 1e-7 and abs(p[0, 1] - 0.25) < 1e-7
    # k = E without renormalization is the full softmax, summing to 1
    rng = np.random.default_rng(3)
    l = rng.standard_normal((50, 8)).astype(np.float32)
    _, p = oracle.router_topk(l, 8, renormalize=False)
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-6)


@pytest.mark.parametrize("renorm", [True, False])
def test_topk_brute_force(renorm):
    rng = np.random.default_rng(5)
    # small integer scores: many exact ties
    l = rng.integers(-3, 4, size=(200, 12)).astype(np.float32)
    k = 5
    ids, p = oracle.router_topk(l, k, renormalize=renorm)
    for t in range(l.shape[0]):
        order = sorted(range(12), key=lambda e: (-float(l[t, e]), e))[:k]
        assert ids[t].tolist() == order
        top = float(l[t, order[0]])
        terms = [math.exp(float(l[t, e]) - top) for e in (order if renorm else range(12))]
        den = math.fsum(terms)
        want = [np.float32(math.exp(float(l[t, e]) - top) / den) for e in order]
        assert np.allclose(p[t], want, rtol=1e-7, atol=0)


def test_topk_matches_the_workload_router():
    rng = np.random.default_rng(7)
    l = rng.standard_normal((500, 128)).astype(np.float32)
    ids, p = oracle.router_topk(l, 8)
    ids_w, p_w = W.route_topk(l, 8)
    assert np.array_equal(ids, ids_w)
    assert np.allclose(p, p_w, rtol=1e-6, atol=0)
