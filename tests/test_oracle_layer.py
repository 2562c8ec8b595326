"""Pins of the oracle's GEMM epilogue, producer, combine, expert sort and layer
wiring against exact arithmetic, closed forms and special cases.  No GPU.

Passages followed: the miniTE summary page, sections "how it differs" (FP32
epilogue multiplies by g^x and g^w, then casts to BF16; router probability on
the SwiGLU activation before FC2; combine order preserved) and "how to use it"
(sort by expert, device offsets for expert boundaries, FC2 maxima from the
router-weighted producer); the article, section 4.4 (SiLU(gate) x up computed
in FP32 and rounded once) and 4.5 (owner sums expert outputs in FP32 in top-k
slot order)."""
import math
from fractions import Fraction

import numpy as np
import pytest

import moe_workloads as W
from tests.exact import (bf16_bits_to_frac, f32_to_frac, frac_to_bf16_bits, near_bf16_boundary)


def _q(orc, x, mode=0):
    return orc.quantize(x, mode)


# --- GEMM + epilogue against exact rational arithmetic ----------------------------------------------

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_gemm_epilogue_exact_bruteforce(orc, seed):
    rng = np.random.default_rng(seed)
    M, N, K = 3, 5, 48
    x = W.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32) * 3)
    w = W.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    xc, xs, gx = _q(orc, x)
    wc, ws, gw = _q(orc, w)
    A = orc.dequantize(xc, xs)
    B = orc.dequantize(wc, ws)
    got = orc.gemm_epilogue(A, gx, B, gw)
    lin = orc.linear((xc, xs, gx), (wc, ws, gw))
    assert np.array_equal(got, lin)
    boundary = 0
    for m in range(M):
        for n in range(N):
            acc = sum(Fraction(float(A[m, k])) * Fraction(float(B[n, k])) for k in range(K))
            exact = acc * f32_to_frac(gx[m]) * f32_to_frac(gw[n])
            if near_bf16_boundary(exact):
                boundary += 1
                continue
            assert int(got[m, n]) == frac_to_bf16_bits(exact), (m, n)
    assert boundary == 0


def test_transparent_inputs_reduce_fc1_to_textbook_matmul(orc):
    """Rows on the E2M1 grid with a 6 in every block quantize to themselves
    (s = 448, fl32(s g) = 1), so the layer's GEMM is the plain matmul of the
    raw values (up to g's own rounding, far below BF16 resolution)."""
    rng = np.random.default_rng(4)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], np.float32)
    M, N, K = 8, 12, 64
    xv = rng.choice(grid, (M, K))
    wv = rng.choice(grid, (N, K))
    xv[:, ::16] = 6
    wv[:, 3::16] = -6
    x, w = W.f32_to_bf16_bits(xv), W.f32_to_bf16_bits(wv)
    xc, xs, gx = _q(orc, x)
    wc, ws, gw = _q(orc, w)
    assert np.all(xs == 0x7E) and np.all(ws == 0x7E)
    A = orc.dequantize(xc, xs)
    assert np.array_equal(A, xv.astype(np.float64) * 448.0)
    out = orc.gemm_epilogue(A, gx, orc.dequantize(wc, ws), gw)
    ref = xv.astype(np.float64) @ wv.astype(np.float64).T  # textbook matmul, exact in FP64
    for m in range(M):
        for n in range(N):
            exact = Fraction(float(ref[m, n]))
            if near_bf16_boundary(exact, rel=2.0 ** -20):
                continue
            assert int(out[m, n]) == frac_to_bf16_bits(exact), (m, n, ref[m, n])


# --- router-weighted SwiGLU producer -----------------------------------------------------------------

def test_silu_closed_forms(orc):
    assert orc.silu(0.0) == 0.0
    assert orc.silu(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)
    for a in (0.1, 1.0, 2.5, 7.0, 30.0, 80.0):
        assert orc.silu(a) - orc.silu(-a) == pytest.approx(a, rel=1e-14)
    assert orc.silu(800.0) == 800.0 and orc.silu(-800.0) == 0.0


def test_swiglu_prob_special_values(orc):
    I = 32
    rng = np.random.default_rng(9)
    vals = W.f32_to_bf16_bits(rng.standard_normal((4, 2 * I)).astype(np.float32))
    y1 = vals.copy()
    y1[0, :I] = 0          # gate 0 -> h = 0
    y1[1, I:] = 0          # up 0   -> h = 0
    p = np.array([0.7, 0.3, 0.0, 1.0], np.float32)  # p 0 -> h = 0
    h, amax2 = orc.swiglu_prob(y1, p)
    hv = W.bf16_bits_to_f32(h)
    assert np.all(hv[0] == 0) and np.all(hv[1] == 0) and np.all(hv[2] == 0)
    assert amax2[0] == 0 and amax2[1] == 0 and amax2[2] == 0
    assert amax2[3] == np.abs(hv[3]).max()
    # one rounding: gate = ln 3 (as BF16), up = 4, p = 1 -> h = bf16(silu(g) * 4) computed exactly enough
    g = W.f32_to_bf16_bits(np.array([math.log(3.0)], np.float32))[0]
    row = np.zeros((1, 2 * I), np.uint16)
    row[0, 0] = g
    row[0, I] = W.f32_to_bf16_bits(np.array([4.0], np.float32))[0]
    h1, _ = orc.swiglu_prob(row, np.array([1.0], np.float32))
    gv = float(bf16_bits_to_frac(g))
    want = gv / (1 + math.exp(-gv)) * 4.0
    assert int(h1[0, 0]) == frac_to_bf16_bits(Fraction(want))


# --- combine in FP32 slot order ------------------------------------------------------------------

def test_combine_k1_is_identity(orc):
    rng = np.random.default_rng(1)
    y = W.f32_to_bf16_bits(rng.standard_normal((5, 1, 64)).astype(np.float32))
    assert np.array_equal(orc.combine(y)[:, :], y[:, 0, :])


def test_combine_is_sequential_fp32_in_slot_order(orc):
    b = lambda v: int(W.f32_to_bf16_bits(np.array([v], np.float32))[0])
    # (256 + 2^-20) rounds back to 256 in FP32, then - 256 = 0; in the other order the tiny term survives.
    y = np.array([[[b(256.0)], [b(2.0 ** -20)], [b(-256.0)]],
                  [[b(256.0)], [b(-256.0)], [b(2.0 ** -20)]]], np.uint16)
    out = orc.combine(y)
    assert int(out[0, 0]) == 0
    assert int(out[1, 0]) == b(2.0 ** -20)
    # an FP32 sum rounded once to BF16 (not a BF16 running sum): 1 + 2^-9 + 2^-9 = 1 + 2^-8 exactly
    y = np.array([[[b(1.0)], [b(2.0 ** -9)], [b(2.0 ** -9)]]], np.uint16)
    assert int(orc.combine(y)[0, 0]) == b(1.0 + 2.0 ** -8)


# --- expert sort layout ----------------------------------------------------------------------------

def test_route_hand_example(orc):
    ids = np.array([[1, 0], [0, 2], [1, 2]], np.int32)
    off, pair2row, row2pair = orc.route(ids, 3, 4)
    assert off.tolist() == [0, 4, 8, 12]
    assert pair2row.tolist() == [4, 0, 1, 8, 5, 9]
    assert row2pair.tolist() == [1, 2, -1, -1, 0, 4, -1, -1, 3, 5, -1, -1]


def test_route_properties(orc):
    wl = W.skewed(T=512)
    E, A = wl.shape.E, 32
    off, pair2row, row2pair = orc.route(wl.ids, E, A)
    cnt = wl.expert_counts()
    assert np.all(np.diff(off) == (cnt + A - 1) // A * A)
    ids = wl.ids.reshape(-1)
    for e in range(E):
        rows = pair2row[ids == e]
        assert np.array_equal(rows, np.arange(off[e], off[e] + cnt[e]))  # stable, packed at the start
    assert np.array_equal(row2pair[pair2row], np.arange(ids.size))
    assert np.sum(row2pair >= 0) == ids.size
    with pytest.raises(ValueError):
        orc.route(np.array([[0, 9]], np.int32), 8, 32)


def test_route_masked_hand_example(orc):
    """Masked fixed-capacity layout (article, section 4.4: per-expert chunks of
    a fixed capacity), worked by hand.  Pairs p = t*K + k of ids below go to
    expert 0: p = 1, 4, 7; expert 1: p = 3; expert 2: p = 0, 2, 5, 6."""
    ids = np.array([[2, 0], [2, 1], [0, 2], [2, 0]], np.int32)
    off, p2r, r2p, used, dropped = orc.route_masked(ids, 3, 2, 4)
    assert off.tolist() == [0, 4, 8, 12] and dropped == 0
    assert p2r.tolist() == [8, 0, 9, 4, 1, 10, 11, 2]
    #                 expert 0 chunk    expert 1 chunk     expert 2 chunk
    assert r2p.tolist() == [1, 4, 7, -1, 3, -1, -1, -1, 0, 2, 5, 6]
    assert used.tolist() == [1, 1, 1, 1, 1, 1, 0, 0, 1, 1, 1, 1]
    # capacity 2: the third and later pairs of an expert get no row
    off, p2r, r2p, used, dropped = orc.route_masked(ids, 3, 2, 2)
    assert off.tolist() == [0, 2, 4, 6] and dropped == 3
    assert p2r.tolist() == [4, 0, 5, 2, 1, -1, -1, -1]
    assert r2p.tolist() == [1, 4, 3, -1, 0, 2]
    assert used.tolist() == [1, 1, 1, 1, 1, 1]
    with pytest.raises(ValueError):
        orc.route_masked(ids, 3, 2, 3)  # not a multiple of m_align
    with pytest.raises(ValueError):
        orc.route_masked(np.array([[0, 3]], np.int32), 3, 2, 4)


def test_route_masked_matches_contiguous_order(orc):
    """With a capacity that holds every expert, each expert's rows are the
    contiguous layout's rows moved to the start of its chunk (same order)."""
    wl = W.skewed(T=512)
    E, A = wl.shape.E, 32
    off_c, p2r_c, _ = orc.route(wl.ids, E, A)
    cap = int(np.diff(off_c).max())
    off, p2r, r2p, used, dropped = orc.route_masked(wl.ids, E, A, cap)
    assert dropped == 0 and np.array_equal(off, np.arange(E + 1) * cap)
    e = wl.ids.reshape(-1)
    assert np.array_equal(p2r, e * cap + (p2r_c - off_c[e]))
    assert np.array_equal(r2p[p2r], np.arange(e.size))
    cnt = wl.expert_counts()
    pad = (cnt + A - 1) // A * A
    assert np.array_equal(used.reshape(E, cap).sum(axis=1), pad)
    # a smaller capacity keeps each expert's first pairs, in the same order
    cap2 = 64
    off, p2r2, r2p2, used2, dropped2 = orc.route_masked(wl.ids, E, A, cap2)
    rank = p2r_c - off_c[e]
    assert dropped2 == int((rank >= cap2).sum()) > 0
    assert np.array_equal(p2r2[rank < cap2], e[rank < cap2] * cap2 + rank[rank < cap2])
    assert np.all(p2r2[rank >= cap2] == -1)


# --- the layer ---------------------------------------------------------------------------------------

def _tiny_layer(seed=0, T=6, H=64, E=3, K=2, I=32):
    wl = W.MoEWorkload("t", seed, W.MoEShape(T=T, H=H, E=E, K=K, I=I))
    w1, w2 = wl.weights(threads=1)
    return wl, w1, w2


def test_layer_wiring_matches_pinned_primitives(orc):
    """moe_forward equals the composition, per (token, slot), of the separately
    pinned primitives, written here from the pages' description."""
    wl, w1, w2 = _tiny_layer()
    T, H, E, K, I = wl.shape.T, wl.shape.H, wl.shape.E, wl.shape.K, wl.shape.I
    wts = orc.DequantWeights(w1, w2)
    out, mid = orc.moe_forward(wl.x, wl.ids, wl.probs, wts, intermediates=True)
    xc, xs, gx = orc.quantize(wl.x)
    Xd = orc.dequantize(xc, xs)
    y2_pairs = np.zeros((T, K, H), np.uint16)
    for t in range(T):
        for k in range(K):
            e = int(wl.ids[t, k])
            rows1 = slice(e * 2 * I, (e + 1) * 2 * I)
            y1 = orc.gemm_epilogue(Xd[t:t + 1], gx[t:t + 1], wts.d1[rows1], wts.g1[rows1])
            assert np.array_equal(y1[0], mid["y1"][t * K + k])
            h, amax2 = orc.swiglu_prob(y1, wl.probs[t:t + 1, k])
            assert np.array_equal(h[0], mid["h"][t * K + k]) and amax2[0] == mid["amax2"][t * K + k]
            hc, hs, gh = orc.quantize(h)
            rows2 = slice(e * H, (e + 1) * H)
            y2 = orc.gemm_epilogue(orc.dequantize(hc, hs), gh, wts.d2[rows2], wts.g2[rows2])
            assert np.array_equal(y2[0], mid["y2"][t * K + k])
            y2_pairs[t, k] = y2[0]
    assert np.array_equal(out, orc.combine(y2_pairs))


def test_fc2_stage_exact_bruteforce(orc):
    """moe_fc2 (FC2 alone from a given h) against exact rationals: Q(h) per
    pair, dequantized values, sum over k, times g^h g^w2, one BF16 rounding;
    and on the layer's own h it returns the layer's y2 bit for bit (both
    routings of the activations: quantized for NVFP4, BF16 for W4A16)."""
    wl, w1, w2 = _tiny_layer(seed=3, T=4, H=32, E=3, K=2, I=32)
    wts = orc.DequantWeights(w1, w2)
    out, mid = orc.moe_forward(wl.x, wl.ids, wl.probs, wts, intermediates=True)
    y2 = orc.moe_fc2(mid["h"], wl.ids, wts)
    assert np.array_equal(y2, mid["y2"])
    H, I = wl.shape.H, wl.shape.I
    e_of = wl.ids.reshape(-1)
    boundary = 0
    for p in range(e_of.size):
        hc, hs, gh = orc.quantize(mid["h"][p:p + 1])
        a = orc.dequantize(hc, hs)[0]
        e = int(e_of[p])
        for m in range(H):
            acc = sum(Fraction(float(a[k])) * Fraction(float(wts.d2[e * H + m, k])) for k in range(I))
            exact = acc * f32_to_frac(gh[0]) * f32_to_frac(wts.g2[e * H + m])
            if near_bf16_boundary(exact):
                boundary += 1
                continue
            assert int(y2[p, m]) == frac_to_bf16_bits(exact), (p, m)
    assert boundary == 0
    # W4A16: FC2 on the BF16 h itself
    out16, mid16 = orc.moe_forward_w4a16(wl.x, wl.ids, wl.probs, wts, intermediates=True)
    y2b = orc.moe_fc2(mid16["h"], wl.ids, wts, quantize_h=False)
    assert np.array_equal(y2b, mid16["y2"])
    p, m = 5, 7
    e = int(e_of[p])
    exact = sum(bf16_bits_to_frac(mid16["h"][p, k]) * Fraction(float(wts.d2[e * H + m, k])) for k in range(I))
    exact *= f32_to_frac(wts.g2[e * H + m])
    assert near_bf16_boundary(exact) or int(y2b[p, m]) == frac_to_bf16_bits(exact)


def test_layer_tokens_are_independent(orc):
    wl, w1, w2 = _tiny_layer(seed=1, T=8)
    wts = orc.DequantWeights(w1, w2)
    out = orc.moe_forward(wl.x, wl.ids, wl.probs, wts)
    perm = np.random.default_rng(0).permutation(8)
    out_p = orc.moe_forward(wl.x[perm], wl.ids[perm], wl.probs[perm], wts)
    assert np.array_equal(out_p, out[perm])
    single = orc.moe_forward(wl.x[3:4], wl.ids[3:4], wl.probs[3:4], wts)
    assert np.array_equal(single[0], out[3])


def test_layer_close_to_unquantized_fp64_moe(orc):
    """Information-level check: the NVFP4 layer tracks the unquantized FP64 MoE
    (the quantization error is a property of the format, so the bound is loose:
    Q alone leaves about 10% relative RMS error on Gaussian rows, each GEMM
    operand carries that, and SwiGLU multiplies the gate and up errors)."""
    wl, w1, w2 = _tiny_layer(seed=2, T=16, H=128, E=4, K=2, I=64)
    wts = orc.DequantWeights(w1, w2)
    out = W.bf16_bits_to_f32(orc.moe_forward(wl.x, wl.ids, wl.probs, wts)).astype(np.float64)
    xv = W.bf16_bits_to_f32(wl.x).astype(np.float64)
    ref = np.zeros_like(out)
    I = wl.shape.I
    for t in range(wl.shape.T):
        for k in range(wl.shape.K):
            e = wl.ids[t, k]
            y1 = W.bf16_bits_to_f32(w1[e]).astype(np.float64) @ xv[t]
            h = y1[:I] / (1 + np.exp(-y1[:I])) * y1[I:] * wl.probs[t, k]
            ref[t] += W.bf16_bits_to_f32(w2[e]).astype(np.float64) @ h
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 0.4, rel
