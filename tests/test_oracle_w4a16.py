"""Pins of the oracle's W4A16 layer (the article, section 6: NVFP4 W4A16 routed
experts -- NVFP4 weights, BF16 activations left unquantized).  No GPU.

  - FC1 and FC2 against exact rational arithmetic on a tiny layer (each
    result is one RNE rounding of sum(x * w_deq) * g^w; the producer and the
    combine are the separately pinned primitives);
  - on activations that the NVFP4 quantizer represents exactly (every block
    on the E2M1 x E4M3 grid, the row's outer scale a power of two), FC1 and
    the producer give the same bits as the W4A4 layer;
  - tokens are independent of their neighbours."""
from fractions import Fraction

import numpy as np

import moe_workloads as W
from tests.exact import bf16_bits_to_frac, f32_to_frac, frac_to_bf16_bits, near_bf16_boundary


def _tiny(seed=0, T=4, H=64, E=3, K=2, I=32):
    wl = W.MoEWorkload("w4a16", seed, W.MoEShape(T=T, H=H, E=E, K=K, I=I))
    w1, w2 = wl.weights(threads=1)
    return wl, w1, w2


def test_w4a16_layer_exact_bruteforce(orc):
    wl, w1, w2 = _tiny()
    T, H, K, I = wl.shape.T, wl.shape.H, wl.shape.K, wl.shape.I
    wts = orc.DequantWeights(w1, w2)
    out, mid = orc.moe_forward_w4a16(wl.x, wl.ids, wl.probs, wts, intermediates=True)
    boundary = 0
    y2_pairs = np.zeros((T, K, H), np.uint16)
    for t in range(T):
        xf = [bf16_bits_to_frac(int(b)) for b in wl.x[t]]
        for k in range(K):
            p, e = t * K + k, int(wl.ids[t, k])
            y1 = np.zeros((1, 2 * I), np.uint16)
            for n in range(2 * I):
                r = e * 2 * I + n
                exact = sum(xf[j] * Fraction(float(wts.d1[r, j])) for j in range(H)) * f32_to_frac(wts.g1[r])
                boundary += near_bf16_boundary(exact)
                y1[0, n] = frac_to_bf16_bits(exact)
            h, _ = orc.swiglu_prob(y1, wl.probs[t:t + 1, k])
            assert np.array_equal(h[0], mid["h"][p]), (t, k)
            hf = [bf16_bits_to_frac(int(b)) for b in h[0]]
            for m in range(H):
                r = e * H + m
                exact = sum(hf[j] * Fraction(float(wts.d2[r, j])) for j in range(I)) * f32_to_frac(wts.g2[r])
                boundary += near_bf16_boundary(exact)
                assert int(mid["y2"][p, m]) == frac_to_bf16_bits(exact), (t, k, m)
            y2_pairs[t, k] = mid["y2"][p]
    assert boundary == 0
    assert np.array_equal(out, orc.combine(y2_pairs))


def _grid_rows(rng, T, H, log2g):
    """BF16 rows the NVFP4 quantizer represents exactly: each 16-element block is
    E2M1 codes times one E4M3 scale times g = 2^log2g, with a 6 in every block,
    and one block per row at scale 448, so max|row| = 6 * 448 * g."""
    e2m1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    e4m3 = np.array([2.0 ** e * (1 + m / 8) for e in range(-6, 8) for m in range(8) if 2.0 ** e * (1 + m / 8) <= 448])
    x = np.zeros((T, H))
    for t in range(T):
        for b in range(H // 16):
            c = rng.choice(e2m1, 16) * rng.choice([-1, 1], 16)
            c[rng.integers(16)] = 6.0 * rng.choice([-1, 1])
            s = 448.0 if b == t % (H // 16) else rng.choice(e4m3)
            x[t, 16 * b:16 * (b + 1)] = c * s * 2.0 ** log2g
    bits = W.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(bits).astype(np.float64), x)  # exact in BF16
    return bits


def test_w4a16_equals_w4a4_on_lossless_activations(orc):
    wl, w1, w2 = _tiny(seed=3, T=5, H=64, E=2, K=2, I=32)
    x = _grid_rows(np.random.default_rng(1), 5, 64, -9)
    c, s, g = orc.quantize(x)
    assert np.all(g == np.float32(2.0 ** -9))
    assert np.array_equal(orc.dequantize(c, s) * 2.0 ** -9, W.bf16_bits_to_f32(x).astype(np.float64))
    wts = orc.DequantWeights(w1, w2)
    _, mid4 = orc.moe_forward(x, wl.ids, wl.probs, wts, intermediates=True)
    _, mid16 = orc.moe_forward_w4a16(x, wl.ids, wl.probs, wts, intermediates=True)
    assert np.array_equal(mid16["h"], mid4["h"])


def test_w4a16_tokens_are_independent(orc):
    wl, w1, w2 = _tiny(seed=4, T=7)
    wts = orc.DequantWeights(w1, w2)
    out = orc.moe_forward_w4a16(wl.x, wl.ids, wl.probs, wts)
    perm = np.random.default_rng(2).permutation(7)
    assert np.array_equal(orc.moe_forward_w4a16(wl.x[perm], wl.ids[perm], wl.probs[perm], wts), out[perm])
    assert np.array_equal(orc.moe_forward_w4a16(wl.x[2:3], wl.ids[2:3], wl.probs[2:3], wts)[0], out[2])
