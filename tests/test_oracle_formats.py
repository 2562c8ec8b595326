"""Pins of the oracle's format helpers and quantizer Q against what the pages
and the format definitions fix (miniTE summary page, section "how it differs":
E2M1 codes, length-16 E4M3 block scales, per-row FP32 outer scale
g = max|row|/(6*448), no stochastic rounding; the article, section 4.4:
elementwise round-to-nearest).  No GPU needed."""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

from tests.exact import frac_to_bf16_bits
from tests.helpers import code_tie_rows, scale_tie_rows, unpack_codes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_hand_cases.json")


def _bf16(v: float) -> int:
    b = struct.unpack("<I", struct.pack("<f", v))[0]
    assert b & 0xFFFF == 0, f"{v} is not a BF16 value"
    return b >> 16


def _f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


# --- format tables ----------------------------------------------------------------------------------

def test_e2m1_values(orc):
    # E2M1 magnitudes from the format (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert orc.e2m1_value(c) == mags[c]
        assert orc.e2m1_value(c | 8) == -mags[c]
        assert math.copysign(1.0, orc.e2m1_value(8)) == -1.0


def test_e4m3_anchor_values(orc):
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x02: 2.0 ** -8, 0x03: 3 * 2.0 ** -9, 0x07: 7 * 2.0 ** -9,
               0x08: 2.0 ** -6, 0x38: 1.0, 0x69: 72.0, 0x6A: 80.0, 0x77: 240.0, 0x7E: 448.0, 0xFE: -448.0}
    for b, v in anchors.items():
        assert orc.e4m3_value(b) == v, hex(b)
    assert math.isnan(orc.e4m3_value(0x7F)) and math.isnan(orc.e4m3_value(0xFF))
    vals = [orc.e4m3_value(b) for b in range(0x7F)]
    assert all(a < b for a, b in zip(vals, vals[1:])), "non-negative E4M3FN codes must increase"
    # every finite value has at most 4 significant bits and lies in [2^-9, 448]
    for v in vals[1:]:
        m, e = math.frexp(v)
        assert (m * 16) == int(m * 16)
        assert 2.0 ** -9 <= v <= 448.0


def test_bf16_rounding_matches_exact(orc):
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(400) * 10.0 ** rng.integers(-45, 38, 400))
    # exact midpoints, their neighbours, subnormals and overflow
    for e in (-130, -127, -20, 0, 5, 127):
        for m in (1, 3, 129, 255):
            base = math.ldexp(m, e)
            half = math.ldexp(1, e - 8 if m > 1 else e - 8)
            xs += [base + half, base - half, math.nextafter(base + half, 0), math.nextafter(base + half, math.inf)]
    xs += [math.ldexp(1, -134), math.ldexp(3, -135), math.ldexp(1, -140), 3.3895313892515355e38, 3.4e38, -2.5e-39]
    for x in xs:
        got = orc.f64_to_bf16(x)
        want = frac_to_bf16_bits(Fraction(x), negative_zero=math.copysign(1, x) < 0)
        assert got == want, (x, hex(got), hex(want))


# --- E2M1 round-to-nearest-even with saturation ------------------------------------------------------

def test_e2m1_encode_ties_and_neighbours(orc):
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(7):
        lo, hi = mags[c], mags[c + 1]
        mid = np.float32((lo + hi) / 2)
        even = c if c % 2 == 0 else c + 1
        assert orc.e2m1_encode(mid) == even, (lo, hi)
        assert orc.e2m1_encode(np.nextafter(mid, np.float32(0))) == c
        assert orc.e2m1_encode(np.nextafter(mid, np.float32(np.inf))) == c + 1
        assert orc.e2m1_encode(np.float32(lo)) == c
    for q in (6.0, 6.5, 7.0, 1e30, float("inf")):
        assert orc.e2m1_encode(q) == 7
    assert orc.e2m1_encode(0.0) == 0


# --- E4M3 block-scale encoders --------------------------------------------------------------------

def test_e4m3_round_up_and_rne(orc):
    vals = [orc.e4m3_value(b) for b in range(0x7F)]
    for b in range(1, 0x7F):
        lo, hi = np.float32(vals[b - 1]), np.float32(vals[b])
        assert orc.e4m3_encode(hi, 0) == b
        assert orc.e4m3_encode(np.nextafter(lo, np.float32(np.inf)), 0) == b
        assert orc.e4m3_encode(hi, 1) == b
        mid = np.float32((vals[b - 1] + vals[b]) / 2)  # exact in binary32
        assert float(mid) == (vals[b - 1] + vals[b]) / 2
        even = b - 1 if (b - 1) % 2 == 0 else b
        assert orc.e4m3_encode(mid, 1) == even
        assert orc.e4m3_encode(np.nextafter(mid, np.float32(0)), 1) == b - 1
        assert orc.e4m3_encode(np.nextafter(mid, np.float32(np.inf)), 1) == b
    for v in (448.0, 448.00003, 500.0, 1e9):
        assert orc.e4m3_encode(v, 0) == 0x7E and orc.e4m3_encode(v, 1) == 0x7E
    assert orc.e4m3_encode(1e-6, 0) == 0x01 and orc.e4m3_encode(1e-6, 1) == 0x00
    assert orc.e4m3_encode(0.0, 0) == 0 and orc.e4m3_encode(0.0, 1) == 0


def test_quantizer_scale_decisions_through_rows(orc):
    """The whole row path (amax, g, 6 g, v, encoder) at every E4M3 decision
    point: with a row maximum of 448, 6 g is exactly 1, so each block's scale
    input is its BF16 maximum; the expected codes follow from the format alone
    (exact values keep their code; at a midpoint RU takes the upper code and
    RNE the even one; a BF16 step either side decides by nearest)."""
    x, want = scale_tie_rows()
    g = np.float32(448) / np.float32(2688)
    assert np.float32(6) * g == np.float32(1)
    for mode in (0, 1):
        _, sc, gg = orc.quantize(x, mode)
        assert np.array_equal(sc, want[mode]), f"mode {mode}: {np.argwhere(sc != want[mode])[:5].tolist()}"
        assert np.all(gg == g)


def test_quantizer_code_decisions_through_rows(orc):
    """The whole row path at every E2M1 decision point under every E4M3
    scale: with a row maximum of 2688, g is exactly 1 and a block whose
    maximum is 6 S gets the scale S, so theta * S (theta an E2M1 midpoint)
    divides back to theta exactly; ties go to the even code, the BF16 values
    beside them to the nearer code, and the sign bit is kept."""
    x, want = code_tie_rows()
    for mode in (0, 1):
        c, _, g = orc.quantize(x, mode)
        assert np.all(g == np.float32(1))
        got = unpack_codes(c)
        assert np.array_equal(got, want), f"mode {mode}: {np.argwhere(got != want)[:5].tolist()}"


# --- Q: hand cases -----------------------------------------------------------------------------------

def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("mode", ["ru", "rne"])
def test_quantizer_hand_cases(orc, case, mode):
    x = np.array([[_bf16(float(v)) for v in case["x"]]], np.uint16)
    codes, scales, g = orc.quantize(x, 0 if mode == "ru" else 1)
    want = case[mode]
    assert [int(c) for c in codes[0]] == [int(c, 16) for c in want["codes"]]
    assert [int(s) for s in scales[0]] == [int(s, 16) for s in want["scales"]]
    assert _f32_bits(g[0]) == int(want["g"], 16)


# --- Q: invariants -----------------------------------------------------------------------------------

def _rows(seed=5, rows=64, cols=256):
    rng = np.random.default_rng(seed)
    import moe_workloads as W
    blocks = []
    blocks.append(rng.standard_normal((rows, cols)))
    x = rng.standard_normal((rows, cols))
    x[rng.random((rows, cols)) < 0.01] *= 50
    blocks.append(x)
    blocks.append(rng.standard_normal((rows, cols)) * 10.0 ** rng.integers(-12, 12, (rows, 1)))
    # per-block dynamic range: some blocks far below the row max (subnormal scales)
    y = rng.standard_normal((rows, cols))
    y *= 10.0 ** rng.integers(-9, 1, (rows, cols // 16)).repeat(16, axis=1)
    blocks.append(y)
    sparse = rng.standard_normal((rows, cols))
    sparse[rng.random((rows, cols)) < 0.7] = 0.0
    blocks.append(sparse)
    return W.f32_to_bf16_bits(np.concatenate(blocks).astype(np.float32))


def _unpack(codes):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


@pytest.mark.parametrize("mode", [0, 1])
def test_quantizer_invariants(orc, mode):
    import moe_workloads as W
    x = _rows()
    codes, scales, g = orc.quantize(x, mode)
    c = _unpack(codes)
    xv = W.bf16_bits_to_f32(x).astype(np.float64)
    mag = np.array([orc.e2m1_value(i) for i in range(16)])
    svals = np.array([orc.e4m3_value(b) for b in range(256)])
    # |code| <= 6 and sign bit equals the input's sign bit
    assert np.all(np.abs(mag[c]) <= 6)
    assert np.array_equal(c >> 3, (x >> 15).astype(np.uint8))
    s = svals[scales]
    bmax = np.abs(xv).reshape(x.shape[0], -1, 16).max(axis=2)
    if mode == 0:
        # scale * 6 * g covers the block amax (up to g's own FP32 rounding)
        cover = s * 6.0 * g[:, None].astype(np.float64)
        assert np.all(cover >= bmax * (1 - 2.0 ** -22))
    # a block whose scale is a normal E4M3 value holds a code of magnitude 6
    cb = (c & 7).reshape(x.shape[0], -1, 16)
    normal = (scales & 0x78) != 0
    assert np.all(cb.max(axis=2)[normal] == 7)
    # rows are independent
    c2, s2, g2 = orc.quantize(x[::-1].copy(), mode)
    assert np.array_equal(c2[::-1], codes) and np.array_equal(s2[::-1], scales) and np.array_equal(g2[::-1], g)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("k", [-10, 3, 20])
def test_quantizer_power_of_two_invariance(orc, mode, k):
    import moe_workloads as W
    x = _rows(seed=6, rows=16)
    xv = W.bf16_bits_to_f32(x)
    keep = np.abs(xv).max(axis=1) < 1e25  # stay inside the binary32 normal range after scaling
    keep &= np.abs(xv).max(axis=1) > 1e-20
    x = x[keep]
    xv = xv[keep]
    xs = W.f32_to_bf16_bits(xv * np.float32(2.0 ** k))
    assert np.array_equal(W.bf16_bits_to_f32(xs), xv * np.float32(2.0 ** k))
    c0, s0, g0 = orc.quantize(x, mode)
    c1, s1, g1 = orc.quantize(xs, mode)
    sub = np.abs(xv).min(axis=1)  # rows whose tiny entries stay normal in both
    assert np.array_equal(c0, c1) and np.array_equal(s0, s1)
    assert np.array_equal(g1, g0 * np.float32(2.0 ** k))


@pytest.mark.parametrize("mode", [0, 1])
def test_quantizer_sign_and_permutation(orc, mode):
    x = _rows(seed=7, rows=16)
    codes, scales, g = orc.quantize(x, mode)
    neg = (x ^ 0x8000).astype(np.uint16)
    cn, sn, gn = orc.quantize(neg, mode)
    assert np.array_equal(sn, scales) and np.array_equal(gn, g)
    assert np.array_equal(_unpack(cn), _unpack(codes) ^ 8)
    rng = np.random.default_rng(3)
    perm = np.concatenate([16 * b + rng.permutation(16) for b in range(x.shape[1] // 16)])
    cp, sp, gp = orc.quantize(x[:, perm].copy(), mode)
    assert np.array_equal(sp, scales) and np.array_equal(gp, g)
    assert np.array_equal(_unpack(cp), _unpack(codes)[:, perm])


def test_dequantize_is_scale_times_code(orc):
    x = _rows(seed=8, rows=4)
    codes, scales, g = orc.quantize(x, 0)
    d = orc.dequantize(codes, scales)
    c = _unpack(codes)
    for r in range(4):
        for j in range(0, x.shape[1], 7):
            assert d[r, j] == orc.e4m3_value(int(scales[r, j // 16])) * orc.e2m1_value(int(c[r, j]))
