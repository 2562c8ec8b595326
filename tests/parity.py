"""Element-wise parity bounds of the GPU path against the oracle.

The oracle accumulates every GEMM in FP64 and rounds once to BF16; the GPU
accumulates exact products (E2M1 x E4M3 values are exact in f16, their
products exact in FP32) in FP32 and rounds fl32(acc * fl32(g_a * g_b)) to
BF16.  For one output element with operand rows a (activation, dequantized
without its outer scale g_a) and b (weight row, likewise, g_b) of length K:

  |acc32 - acc|   <= 2 K u sum_k |a_k b_k| <= 2 K u ||a|| ||b||
                     (any summation order or tree, each addition rounded with
                     relative error <= 2u: covers round-to-nearest and
                     truncating adders; Cauchy-Schwarz for the sum)
  epilogue        two FP32 products: relative error <= 3u of |y|
  BF16 rounding   two values rounded to BF16 differ by at most their
                  distance plus one BF16 ulp of the larger

so |y_gpu - y_ref| <= 2 K u g_a g_b ||a|| ||b|| + 3u |y_ref| + ulp(max(|y_ref|, |y_gpu|))
with u = 2^-24.  A wrong row, column, scale or expert moves an element by
about |y| itself, far beyond this bound (about 1 % of a typical |y| at
K = 2048).

The producer: the GPU forms silu(gate) * up * p in FP32 with the hardware
exp2 and reciprocal (relative error a few FP32 ulps) and rounds once; from
the same gate and up the oracle's FP64 value differs by a relative 1e-6 or
less, so the two BF16 results are equal or one BF16 ulp apart (for gates
above -64, where exp does not overflow: asserted by the callers).

Helpers here only take norms and compare; every expected value comes from
the oracle.
"""
from __future__ import annotations

import numpy as np

import moe_workloads as W

U = 2.0 ** -24  # FP32 unit roundoff


def vals(bits: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


def ulp_bf16(mag: np.ndarray) -> np.ndarray:
    """BF16 spacing at |v| (8 significant bits; subnormal spacing 2^-133)."""
    m = np.abs(np.asarray(mag, np.float64))
    e = np.floor(np.log2(np.maximum(m, 2.0 ** -126)))
    return np.exp2(np.maximum(e - 7, -133))


def ulp_dist(got_bits, ref_bits) -> np.ndarray:
    """|got - ref| in BF16 ulps of the larger magnitude (0 where both are 0)."""
    g, r = vals(got_bits), vals(ref_bits)
    d = np.abs(g - r)
    return np.where(d == 0, 0.0, d / ulp_bf16(np.maximum(np.abs(g), np.abs(r))))


def row_norms(a: np.ndarray) -> np.ndarray:
    return np.sqrt(np.einsum("ij,ij->i", a, a))


class Check:
    """Accumulates element-wise comparisons of one stage; fails with a precise message."""

    def __init__(self, what: str):
        self.what, self.n, self.worst, self.ulp1, self.ulp2, self.max_ulp = what, 0, 0.0, 0, 0, 0.0

    def add(self, got_bits, ref_bits, bound, index_offset=0):
        g, r = vals(got_bits), vals(ref_bits)
        err = np.abs(g - r)
        ratio = err / bound
        bad = np.argwhere(ratio > 1.0 + 1e-9)
        if bad.size:
            i = tuple(bad[0])
            raise AssertionError(f"{self.what}: {bad.shape[0]} elements out of bound; first at "
                                 f"{(i[0] + index_offset,) + i[1:]}: got {g[i]!r} ref {r[i]!r} bound {bound[i]!r}")
        u = ulp_dist(got_bits, ref_bits)
        self.n += err.size
        self.worst = max(self.worst, float(ratio.max()) if ratio.size else 0.0)
        self.ulp1 += int((u > 1).sum())
        self.ulp2 += int((u > 2).sum())
        self.max_ulp = max(self.max_ulp, float(u.max()) if u.size else 0.0)

    def report(self) -> str:
        return (f"{self.what}: {self.n} elements within bound (worst {self.worst:.3f} of it), max {self.max_ulp:.1f} "
                f"BF16 ulps, {self.ulp1} > 1 ulp, {self.ulp2} > 2 ulps")


def gemm_bound(ref_bits, got_bits, a_scaled_norm, b_scaled_norm, K):
    """Bound of |got - ref| per element of y [n_a, n_b] = bf16(acc * g_a * g_b):
    a_scaled_norm [n_a] = g_a ||a||, b_scaled_norm [n_a, n_b] or [n_b] = g_b ||b||."""
    r, g = vals(ref_bits), vals(got_bits)
    acc = 2.0 * K * U * a_scaled_norm[:, None] * b_scaled_norm
    return acc + 3.0 * U * np.abs(r) + ulp_bf16(np.maximum(np.abs(r), np.abs(g)))


def check_grouped_gemm(check: Check, got_bits, ref_bits, a_scaled_norm, b_scaled_norm_rows, expert_of_row, K,
                       chunk=4096):
    """got/ref [R, N]; row i uses activation norm a_scaled_norm[i] and the weight
    rows of expert expert_of_row[i] (b_scaled_norm_rows [E, N])."""
    R = got_bits.shape[0]
    for i0 in range(0, R, chunk):
        sl = slice(i0, min(R, i0 + chunk))
        bnd = gemm_bound(ref_bits[sl], got_bits[sl], a_scaled_norm[sl], b_scaled_norm_rows[expert_of_row[sl]], K)
        check.add(got_bits[sl], ref_bits[sl], bnd, index_offset=i0)


def check_producer(check: Check, got_h, ref_h, y1_bits, I):
    """h from the same y1: equal or one BF16 ulp apart (gates above -64)."""
    gate = vals(y1_bits[:, :I])
    assert gate.size == 0 or gate.min() > -64.0, "producer bound assumes gates above -64"
    for i0 in range(0, got_h.shape[0], 8192):
        sl = slice(i0, min(got_h.shape[0], i0 + 8192))
        g, r = vals(got_h[sl]), vals(ref_h[sl])
        bnd = ulp_bf16(np.maximum(np.abs(g), np.abs(r)))
        check.add(got_h[sl], ref_h[sl], bnd, index_offset=i0)


def combine_bound(y2g_pairs, y2r_pairs, y2_bounds, out_ref_bits, out_got_bits):
    """Bound of |out_gpu - out_ref| for out = bf16(FP32 slot-order sum of y2), the
    y2 of slot k within y2_bounds[:, k] of each other ([T, K, H] arrays): the
    sums differ by the inputs' distances plus both sums' FP32 rounding (each
    partial sum rounded with error <= u |partial| <= u sum |terms|), then one
    BF16 ulp of the larger output."""
    K = y2g_pairs.shape[1]
    mag = np.maximum(np.abs(vals(y2g_pairs)), np.abs(vals(y2r_pairs))).sum(axis=1)
    r, g = vals(out_ref_bits), vals(out_got_bits)
    return y2_bounds.sum(axis=1) + 2.0 * max(K - 1, 0) * U * mag + ulp_bf16(np.maximum(np.abs(r), np.abs(g)))
