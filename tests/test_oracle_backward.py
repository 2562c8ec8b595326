"""Pins of the oracle's BF16 straight-through backward (miniTE summary page,
"how it differs": the backward takes quantization as the identity and runs
BF16 GEMMs on the stored original BF16 activations and weights).  No GPU.

  - silu' against difference quotients of silu, and closed forms;
  - every GEMM-shaped gradient (dh, the FC1 input gradient, dW1, dW2) against
    exact rational sums written here from the chain rule;
  - the whole backward against central differences of an unquantized FP64
    MoE layer (numpy, written here), through which a transposed operand, a
    wrong slot, a missing router factor or a sign error would show;
  - special cases: a zero upstream gradient, a zero router probability."""
import math
from fractions import Fraction

import numpy as np
import pytest

import moe_workloads as W
from tests.exact import bf16_bits_to_frac, frac_to_bf16_bits, near_bf16_boundary


def test_silu_grad_closed_forms_and_difference_quotients(orc):
    assert orc.silu_grad(0.0) == 0.5
    # sigmoid(ln 3) = 3/4: silu'(ln 3) = 3/4 (1 + ln 3 / 4)
    assert abs(orc.silu_grad(math.log(3.0)) - 0.75 * (1 + math.log(3.0) / 4)) < 1e-15
    for a in (-20.0, -6.5, -1.3, -0.2, 0.7, 2.9, 11.0):
        eps = 1e-5 * max(1.0, abs(a))
        fd = (orc.silu(a + eps) - orc.silu(a - eps)) / (2 * eps)
        assert abs(fd - orc.silu_grad(a)) <= 1e-8 * max(1.0, abs(fd)), a


def _case(seed, T=3, H=32, I=16, E=2, K=2):
    rng = np.random.default_rng(seed)
    bf = lambda a: W.f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    x = bf(rng.standard_normal((T, H)))
    w1 = bf(rng.standard_normal((E, 2 * I, H)) * 0.2)
    w2 = bf(rng.standard_normal((E, H, I)) * 0.2)
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    probs = rng.uniform(0.1, 1.0, (T, K)).astype(np.float32)
    y1 = bf(rng.standard_normal((T * K, 2 * I)))
    h = bf(rng.standard_normal((T * K, I)))
    dout = bf(rng.standard_normal((T, H)))
    return x, w1, w2, ids, probs, y1, h, dout


def _v(bits):
    return W.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def test_gemm_gradients_exact(orc):
    """dh, the per-pair FC1 input gradient (K = 1 makes dx equal to it), dW1 and
    dW2 against exact rational sums over the chain rule's terms."""
    x, w1, w2, ids, probs, y1, h, dout = _case(0, T=3, K=1)
    T, H = x.shape
    E, twoI, _ = w1.shape
    I = twoI // 2
    dx, dprobs, dw1, dw2, mid = orc.moe_backward(x, ids, probs, w1, w2, y1, h, dout, intermediates=True)
    boundary = 0
    for p in range(T):
        e = int(ids[p, 0])
        for n in range(I):
            exact = sum(bf16_bits_to_frac(dout[p, m]) * bf16_bits_to_frac(w2[e, m, n]) for m in range(H))
            if near_bf16_boundary(exact):
                boundary += 1
                continue
            assert int(mid["dh"][p, n]) == frac_to_bf16_bits(exact), ("dh", p, n)
        for m in range(H):
            exact = sum(bf16_bits_to_frac(mid["dy1"][p, j]) * bf16_bits_to_frac(w1[e, j, m]) for j in range(twoI))
            if near_bf16_boundary(exact):
                boundary += 1
                continue
            assert int(dx[p, m]) == frac_to_bf16_bits(exact), ("dx", p, m)
    assert boundary == 0
    for e in range(E):
        pairs = [p for p in range(T) if ids[p, 0] == e]
        for j in range(0, twoI, 5):
            for m in range(0, H, 3):
                exact = sum(bf16_bits_to_frac(mid["dy1"][p, j]) * bf16_bits_to_frac(x[p, m]) for p in pairs)
                assert abs(float(dw1[e, j, m]) - float(exact)) <= abs(float(exact)) * 2.0 ** -24, ("dW1", e, j, m)
        for m in range(0, H, 3):
            for n in range(I):
                exact = sum(bf16_bits_to_frac(dout[p, m]) * bf16_bits_to_frac(h[p, n]) for p in pairs)
                assert abs(float(dw2[e, m, n]) - float(exact)) <= abs(float(exact)) * 2.0 ** -24, ("dW2", e, m, n)


def _fp64_layer_loss(x, w1, w2, ids, probs, dout):
    """Unquantized FP64 MoE layer: L = sum_t <dout[t], sum_k W2[e] (silu(g) u p)>."""
    T, H = x.shape
    I = w1.shape[1] // 2
    L = 0.0
    for t in range(T):
        o = np.zeros(H)
        for k in range(ids.shape[1]):
            e = ids[t, k]
            y = w1[e] @ x[t]
            g, u = y[:I], y[I:]
            o += w2[e] @ (g / (1 + np.exp(-g)) * u * probs[t, k])
        L += float(dout[t] @ o)
    return L


def test_backward_matches_difference_quotients_of_the_unquantized_layer(orc):
    """Fed the activations of the unquantized FP64 layer (rounded to BF16), the
    straight-through backward gives that layer's gradient up to the BF16
    roundings of its intermediates; compared with central differences at
    sampled coordinates of x, W1, W2 and the router probabilities."""
    T, H, I, E, K = 4, 24, 16, 3, 2
    x, w1, w2, ids, probs, _, _, dout = _case(7, T=T, H=H, I=I, E=E, K=K)
    xv, w1v, w2v, dv = _v(x), _v(w1), _v(w2), _v(dout)
    pv = probs.astype(np.float64)
    y1 = np.zeros((T * K, 2 * I))
    hh = np.zeros((T * K, I))
    for t in range(T):
        for k in range(K):
            e = ids[t, k]
            y1[t * K + k] = w1v[e] @ xv[t]
    y1b = W.f32_to_bf16_bits(y1.astype(np.float32))
    y1r = _v(y1b)
    for p in range(T * K):
        g, u = y1r[p, :I], y1r[p, I:]
        hh[p] = g / (1 + np.exp(-g)) * u * pv.reshape(-1)[p]
    hb = W.f32_to_bf16_bits(hh.astype(np.float32))
    dx, dprobs, dw1, dw2 = orc.moe_backward(x, ids, probs, w1, w2, y1b, hb, dout)
    rng = np.random.default_rng(3)

    def fd(which, idx, eps=1e-4):
        args = {"x": xv.copy(), "w1": w1v.copy(), "w2": w2v.copy(), "p": pv.copy()}
        args[which][idx] += eps
        lp = _fp64_layer_loss(args["x"], args["w1"], args["w2"], ids, args["p"], dv)
        args[which][idx] -= 2 * eps
        lm = _fp64_layer_loss(args["x"], args["w1"], args["w2"], ids, args["p"], dv)
        return (lp - lm) / (2 * eps)

    checks = [("x", _v(dx), xv.shape), ("w1", dw1.astype(np.float64), w1v.shape),
              ("w2", dw2.astype(np.float64), w2v.shape), ("p", dprobs.astype(np.float64), pv.shape)]
    for which, grad, shape in checks:
        scale = np.sqrt(np.mean(grad ** 2))
        assert scale > 0
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in shape)
            num = fd(which, idx)
            assert abs(grad[idx] - num) <= 3e-2 * scale + 1e-2 * abs(num), (which, idx, grad[idx], num)


def test_special_cases(orc):
    x, w1, w2, ids, probs, y1, h, dout = _case(11, T=3, K=2)
    # zero upstream gradient: every gradient is zero
    z = np.zeros_like(dout)
    dx, dprobs, dw1, dw2 = orc.moe_backward(x, ids, probs, w1, w2, y1, h, z)
    assert not _v(dx).any() and not dprobs.any() and not dw1.any() and not dw2.any()
    # a zero router probability: that pair passes no gradient to FC1 (its dy1 is
    # zero), while its own probability still gets d/dp = <dh, silu(gate) up>
    probs0 = probs.copy()
    probs0[1, 0] = 0.0
    dx0, dp0, dw10, dw20, mid = orc.moe_backward(x, ids, probs0, w1, w2, y1, h, dout, intermediates=True)
    assert not _v(mid["dy1"][2]).any()
    g, u = _v(y1[2, :16]), _v(y1[2, 16:])
    want = float(np.sum(_v(mid["dh"][2]) * (g / (1 + np.exp(-g))) * u))
    assert abs(float(dp0[1, 0]) - want) <= 1e-6 * abs(want)


def test_backward_is_the_composition_of_its_steps(orc):
    """moe_backward equals its steps run one at a time: dh (exact-pinned GEMM),
    swiglu_backward, each pair's FC1 input gradient, the combine, and
    moe_weight_grads."""
    x, w1, w2, ids, probs, y1, h, dout = _case(5, T=5, H=32, I=16, E=3, K=2)
    dx, dprobs, dw1, dw2, mid = orc.moe_backward(x, ids, probs, w1, w2, y1, h, dout, intermediates=True)
    dy1, dprob = orc.swiglu_backward(mid["dh"], y1, probs)
    assert np.array_equal(dy1, mid["dy1"]) and np.array_equal(dprob.view(np.uint32), dprobs.reshape(-1).view(np.uint32))
    g1, g2 = orc.moe_weight_grads(x, dout, ids, mid["dy1"], h, w1.shape[0])
    assert np.array_equal(g1, dw1) and np.array_equal(g2, dw2)
    # FC1 input gradient per pair, then the slot-order combine
    T, K = ids.shape
    dxp = np.zeros((T, K, x.shape[1]), np.uint16)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            dxp[t, k] = orc.gemm_epilogue(_v(mid["dy1"][t * K + k:t * K + k + 1]), np.ones(1, np.float32),
                                          _v(w1[e]).T.copy(), np.ones(x.shape[1], np.float32))[0]
    assert np.array_equal(orc.combine(dxp), dx)
