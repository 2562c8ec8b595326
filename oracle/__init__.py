"""CPU oracle of the NVFP4 MoE expert forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``nvfp4_moe_expert_sort_amd``) never imports it, and the two share no code.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, FP64 GEMMs, one BF16
rounding per result); this module only builds that file with gcc and marshals
numpy arrays into it with ctypes.  Each wrapper names the passage of the pages
it follows: the miniTE summary page ("miniTE diagnoses and narrows the
cross-engine execution gap of NVFP4 RL", sections "how it differs" and "how to
use it") and the article "Finish RL training faster: bitwise consistent,
high-performance, agent-driven", sections 4.4 and 4.5.

Functions whose parity is not pinned by an independent check: none (the
SwiGLU producer is pinned by special values and the identity
silu(a) - silu(-a) = a; beyond those, its transcendental is FP64 ``exp``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

SCALE_RU = 0
SCALE_RNE = 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (IEEE binary32/64 arithmetic, no FMA contraction)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
           "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_bf16_to_double.restype = ctypes.c_double
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_double_to_bf16.restype = ctypes.c_uint16
    lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_e2m1_value.argtypes = [ctypes.c_int]
    lib.orc_e4m3_value.restype = ctypes.c_double
    lib.orc_e4m3_value.argtypes = [ctypes.c_int]
    lib.orc_e2m1_encode.restype = ctypes.c_int
    lib.orc_e2m1_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode.restype = ctypes.c_int
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.orc_silu.restype = ctypes.c_double
    lib.orc_silu.argtypes = [ctypes.c_double]
    lib.orc_quantize.restype = None
    lib.orc_quantize.argtypes = [P, I64, I64, I64, ctypes.c_int, P, P, P]
    lib.orc_dequantize.restype = None
    lib.orc_dequantize.argtypes = [P, P, I64, I64, P]
    lib.orc_gemm_epilogue.restype = None
    lib.orc_gemm_epilogue.argtypes = [P, P, I64, P, P, I64, I64, P]
    lib.orc_linear.restype = None
    lib.orc_linear.argtypes = [P, P, P, I64, P, P, P, I64, I64, P]
    lib.orc_swiglu_prob.restype = None
    lib.orc_swiglu_prob.argtypes = [P, P, I64, I64, P, P]
    lib.orc_combine.restype = None
    lib.orc_combine.argtypes = [P, I64, I64, I64, P]
    lib.orc_route.restype = I64
    lib.orc_route.argtypes = [P, I64, I64, I64, I64, P, P, P, I64]
    lib.orc_router_logits.restype = None
    lib.orc_router_logits.argtypes = [P, I64, I64, P, I64, P]
    lib.orc_router_topk.restype = None
    lib.orc_router_topk.argtypes = [P, I64, I64, I64, ctypes.c_int, P, P]
    lib.orc_moe_forward_deq.restype = None
    lib.orc_moe_forward_deq.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P, ctypes.c_int, P, P, P, P, P]
    lib.orc_moe_forward_w4a16.restype = None
    lib.orc_moe_forward_w4a16.argtypes = [P, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P]
    lib.orc_moe_fc2.restype = None
    lib.orc_moe_fc2.argtypes = [P, I64, I64, I64, P, P, P, ctypes.c_int, ctypes.c_int, P]
    lib.orc_silu_grad.restype = ctypes.c_double
    lib.orc_silu_grad.argtypes = [ctypes.c_double]
    lib.orc_moe_backward.restype = None
    lib.orc_moe_backward.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, P]
    lib.orc_swiglu_backward.restype = None
    lib.orc_swiglu_backward.argtypes = [P, P, P, I64, I64, P, P]
    lib.orc_moe_weight_grads.restype = None
    lib.orc_moe_weight_grads.argtypes = [P, P, I64, I64, I64, I64, I64, P, P, P, P, P]
    lib.orc_route_masked.restype = I64
    lib.orc_route_masked.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P]
    lib.orc_moe_forward.restype = None
    lib.orc_moe_forward.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, ctypes.c_int, P, P, P,
                                    P, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- formats (definitions of E2M1, E4M3FN and BF16) --------------------------------------------------

def bf16_to_f64(bits: int) -> float:
    return _load().orc_bf16_to_double(int(bits))


def f64_to_bf16(x: float) -> int:
    """One RNE rounding of an FP64 value onto the BF16 grid."""
    return int(_load().orc_double_to_bf16(float(x)))


def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().orc_e4m3_value(int(byte))


def e2m1_encode(q: float) -> int:
    """Nearest E2M1 magnitude code to the FP32 value q, ties to even, saturating at 6."""
    return int(_load().orc_e2m1_encode(float(q)))


def e4m3_encode(v: float, mode: int = SCALE_RU) -> int:
    return int(_load().orc_e4m3_encode(float(v), int(mode)))


def silu(a: float) -> float:
    return _load().orc_silu(float(a))


# --- quantizer Q (miniTE page, "how it differs") ------------------------------------------------------

def quantize(x_bf16: np.ndarray, mode: int = SCALE_RU):
    """Q over every row of a [rows, cols] BF16 (uint16) array.

    Returns (codes [rows, cols/2] uint8, low nibble = even element;
    scales [rows, cols/16] uint8 E4M3FN; g [rows] float32)."""
    x = _c(x_bf16, np.uint16)
    rows, cols = x.shape
    assert cols % 16 == 0
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    g = np.empty((rows,), np.float32)
    _load().orc_quantize(_p(x), rows, cols, cols, int(mode), _p(codes), _p(scales), _p(g))
    return codes, scales, g


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """s * E2M1(code) per element in FP64 (exact), without the outer scale g."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rows = codes.shape[0]
    cols = codes.shape[1] * 2
    out = np.empty((rows, cols), np.float64)
    _load().orc_dequantize(_p(codes), _p(scales), rows, cols, _p(out))
    return out


# --- GEMM + FP32-epilogue semantics, producer, combine -------------------------------------------------

def gemm_epilogue(a_deq, ga, b_deq, gb) -> np.ndarray:
    """bf16((A . B^T) * ga[m] * gb[n]); FP64 sum over k ascending, one rounding."""
    A = _c(a_deq, np.float64)
    B = _c(b_deq, np.float64)
    ga = _c(ga, np.float32)
    gb = _c(gb, np.float32)
    M, K = A.shape
    N = B.shape[0]
    out = np.empty((M, N), np.uint16)
    _load().orc_gemm_epilogue(_p(A), _p(ga), M, _p(B), _p(gb), N, K, _p(out))
    return out


def linear(xq, wq) -> np.ndarray:
    """Dense NVFP4 linear from quantized operands (codes, scales, g) of X [M,K] and W [N,K]."""
    xc, xs, gx = (_c(xq[0], np.uint8), _c(xq[1], np.uint8), _c(xq[2], np.float32))
    wc, ws, gw = (_c(wq[0], np.uint8), _c(wq[1], np.uint8), _c(wq[2], np.float32))
    M, K = xc.shape[0], xc.shape[1] * 2
    N = wc.shape[0]
    out = np.empty((M, N), np.uint16)
    _load().orc_linear(_p(xc), _p(xs), _p(gx), M, _p(wc), _p(ws), _p(gw), N, K, _p(out))
    return out


def swiglu_prob(y1: np.ndarray, p: np.ndarray):
    """h = bf16(silu(gate) * up * p) per row of y1 = [gate | up]; returns (h, amax2)."""
    y1 = _c(y1, np.uint16)
    p = _c(p, np.float32)
    R, twoI = y1.shape
    I = twoI // 2
    h = np.empty((R, I), np.uint16)
    amax2 = np.empty((R,), np.float32)
    _load().orc_swiglu_prob(_p(y1), _p(p), R, I, _p(h), _p(amax2))
    return h, amax2


def combine(y2_pairs: np.ndarray) -> np.ndarray:
    """FP32 sum in slot order of y2 given per pair as [T, K, H] BF16; one BF16 rounding."""
    y2 = _c(y2_pairs, np.uint16)
    T, K, H = y2.shape
    out = np.empty((T, H), np.uint16)
    _load().orc_combine(_p(y2), T, K, H, _p(out))
    return out


def route(ids: np.ndarray, n_experts: int, m_align: int):
    """Expected sorted layout: (off [E+1] int64, pair2row [T*K] int32, row2pair [P_pad] int32)."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    off = np.empty((n_experts + 1,), np.int64)
    pair2row = np.empty((T * K,), np.int32)
    cap = T * K + n_experts * m_align
    row2pair = np.empty((cap,), np.int32)
    P_pad = _load().orc_route(_p(ids), T, K, n_experts, m_align, _p(off), _p(pair2row), _p(row2pair), cap)
    if P_pad < 0:
        raise ValueError("expert id out of range")
    return off, pair2row, row2pair[:P_pad].copy()


def silu_grad(a: float) -> float:
    """d silu / d a in FP64."""
    return _load().orc_silu_grad(float(a))


def moe_backward(x_bf16, ids, probs, w1_bf16, w2_bf16, y1, h, dout, intermediates: bool = False):
    """The BF16 straight-through backward of the expert forward (miniTE page,
    "how it differs": straight-through approximation, BF16 GEMMs on the stored
    original BF16 activations and weights).  y1 [P, 2I] and h [P, I] are the
    forward's BF16 FC1 output and FC2 input per pair; dout [T, H] BF16.
    Returns (dx [T, H] BF16 bits, dprobs [T, K] f32, dW1 [E, 2I, H] f32,
    dW2 [E, H, I] f32), plus dict(dh [P, I], dy1 [P, 2I]) with ``intermediates``."""
    x = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    probs = _c(probs, np.float32)
    w1 = _c(w1_bf16, np.uint16)
    w2 = _c(w2_bf16, np.uint16)
    y1 = _c(y1, np.uint16)
    h = _c(h, np.uint16)
    dout = _c(dout, np.uint16)
    T, H = x.shape
    K = ids.shape[1]
    E, twoI, _ = w1.shape
    I = twoI // 2
    assert w2.shape == (E, H, I) and y1.shape == (T * K, 2 * I) and h.shape == (T * K, I) and dout.shape == (T, H)
    if ids.size and (ids.min() < 0 or ids.max() >= E):
        raise ValueError("expert id out of range")
    dx = np.empty((T, H), np.uint16)
    dprobs = np.empty((T, K), np.float32)
    dw1 = np.empty((E, 2 * I, H), np.float32)
    dw2 = np.empty((E, H, I), np.float32)
    dh = np.empty((T * K, I), np.uint16) if intermediates else None
    dy1 = np.empty((T * K, 2 * I), np.uint16) if intermediates else None
    _load().orc_moe_backward(_p(x), T, H, I, E, K, _p(ids), _p(probs), _p(w1), _p(w2), _p(y1), _p(h), _p(dout),
                             _p(dx), _p(dprobs), _p(dw1), _p(dw2), _p(dh), _p(dy1))
    if intermediates:
        return dx, dprobs, dw1, dw2, dict(dh=dh, dy1=dy1)
    return dx, dprobs, dw1, dw2


def swiglu_backward(dh, y1, p):
    """SwiGLU backward per row (the backward's producer step): (dy1 [R, 2I] BF16 bits, dprob [R] f32)."""
    dh = _c(dh, np.uint16)
    y1 = _c(y1, np.uint16)
    p = _c(p, np.float32).reshape(-1)
    R, I = dh.shape
    assert y1.shape == (R, 2 * I) and p.size == R
    dy1 = np.empty((R, 2 * I), np.uint16)
    dprob = np.empty((R,), np.float32)
    _load().orc_swiglu_backward(_p(dh), _p(y1), _p(p), R, I, _p(dy1), _p(dprob))
    return dy1, dprob


def moe_weight_grads(x_bf16, dout, ids, dy1, h, n_experts: int):
    """Weight gradients from given per-pair gradients (the backward's last step):
    (dW1 [E, 2I, H] f32, dW2 [E, H, I] f32), sums over each expert's pairs in
    increasing pair order in FP64."""
    x = _c(x_bf16, np.uint16)
    dout = _c(dout, np.uint16)
    ids = _c(ids, np.int32)
    dy1 = _c(dy1, np.uint16)
    h = _c(h, np.uint16)
    T, H = x.shape
    K = ids.shape[1]
    I = h.shape[1]
    E = int(n_experts)
    dw1 = np.empty((E, 2 * I, H), np.float32)
    dw2 = np.empty((E, H, I), np.float32)
    _load().orc_moe_weight_grads(_p(x), _p(dout), T, H, I, E, K, _p(ids), _p(dy1), _p(h), _p(dw1), _p(dw2))
    return dw1, dw2


def route_masked(ids: np.ndarray, n_experts: int, m_align: int, capacity: int):
    """Expected masked fixed-capacity layout (article, section 4.4, "two layouts,
    same row results"): expert e owns rows [e*capacity, (e+1)*capacity).

    Returns (off [E+1] int64, pair2row [T*K] int32 (-1: no row, past the
    capacity), row2pair [E*capacity] int32 (-1: padding or unused),
    row_used [E*capacity] bool (kept and padding rows), n_dropped)."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    off = np.empty((n_experts + 1,), np.int64)
    pair2row = np.empty((T * K,), np.int32)
    row2pair = np.empty((n_experts * capacity,), np.int32)
    used = np.empty((n_experts * capacity,), np.uint8)
    n = _load().orc_route_masked(_p(ids), T, K, n_experts, m_align, capacity, _p(off), _p(pair2row), _p(row2pair),
                                 _p(used))
    if n == -1:
        raise ValueError("expert id out of range")
    if n == -2:
        raise ValueError("capacity must be a positive multiple of m_align")
    return off, pair2row, row2pair, used.astype(bool), int(n)


def moe_fc2(h_pairs, ids, weights: "DequantWeights", quantize_h: bool = True, mode: int = SCALE_RU):
    """FC2 alone from a given h, one row per pair p = t*K + k (miniTE page, "how
    it differs": FC2 on Q(h) with the same epilogue; quantize_h False: the
    W4A16 variant's unquantized BF16 h).  The arithmetic is the layer's own
    FC2 step.  Returns y2 [P, H] BF16 bits."""
    h = _c(h_pairs, np.uint16)
    ids = _c(ids, np.int32).reshape(-1)
    P, I = h.shape
    assert ids.size == P and I == weights.I
    if ids.size and (ids.min() < 0 or ids.max() >= weights.E):
        raise ValueError("expert id out of range")
    y2 = np.empty((P, weights.H), np.uint16)
    _load().orc_moe_fc2(_p(h), P, I, weights.H, _p(ids), _p(weights.d2), _p(weights.g2), 1 if quantize_h else 0,
                        int(mode), _p(y2))
    return y2


def moe_forward_w4a16(x_bf16, ids, probs, weights: DequantWeights, intermediates: bool = False):
    """The W4A16 variant (article, section 6: NVFP4 W4A16 routed experts): NVFP4
    weights, BF16 activations not quantized; epilogues multiply by g^w only.
    Returns out [T,H] BF16 bits, and with ``intermediates`` per-pair y1 [P,2I], h [P,I], y2 [P,H]."""
    x = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    probs = _c(probs, np.float32)
    T, H = x.shape
    K = ids.shape[1]
    I = weights.I
    assert H == weights.H
    if ids.size and (ids.min() < 0 or ids.max() >= weights.E):
        raise ValueError("expert id out of range")
    P = T * K
    out = np.empty((T, H), np.uint16)
    y1 = np.empty((P, 2 * I), np.uint16) if intermediates else None
    h = np.empty((P, I), np.uint16) if intermediates else None
    y2 = np.empty((P, H), np.uint16) if intermediates else None
    _load().orc_moe_forward_w4a16(_p(x), T, H, I, K, _p(ids), _p(probs), _p(weights.d1), _p(weights.g1),
                                  _p(weights.d2), _p(weights.g2), _p(out), _p(y1), _p(h), _p(y2))
    if intermediates:
        return out, dict(y1=y1, h=h, y2=y2)
    return out


def router_logits(x_bf16: np.ndarray, w_bf16: np.ndarray) -> np.ndarray:
    """Router scores x . w^T of BF16 x [T, H] and w [E, H], exact in FP64 (article,
    section 4.4, "R3 unnecessary": one FP32-output scoring kernel for every batch size)."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_bf16, np.uint16)
    T, H = x.shape
    E = w.shape[0]
    assert w.shape[1] == H
    out = np.empty((T, E), np.float64)
    _load().orc_router_logits(_p(x), T, H, _p(w), E, _p(out))
    return out


def router_topk(logits_f32: np.ndarray, k: int, renormalize: bool = True):
    """Top-k of FP32 router scores: higher score first, equal scores to the lower
    expert id (article, section 2: same tie-breaking and output order); softmax
    probabilities over the k selected (renormalize) or all experts, FP64 -> FP32."""
    l = _c(logits_f32, np.float32)
    T, E = l.shape
    ids = np.empty((T, k), np.int32)
    probs = np.empty((T, k), np.float32)
    _load().orc_router_topk(_p(l), T, E, k, 1 if renormalize else 0, _p(ids), _p(probs))
    return ids, probs


class DequantWeights:
    """Expert weights quantized by the oracle's Q and held dequantized in FP64."""

    def __init__(self, w1_bf16, w2_bf16, mode: int = SCALE_RU):
        E, twoI, H = w1_bf16.shape
        I = twoI // 2
        assert w2_bf16.shape == (E, H, I)
        self.E, self.H, self.I = E, H, I
        c1, s1, self.g1 = quantize(w1_bf16.reshape(E * twoI, H), mode)
        c2, s2, self.g2 = quantize(w2_bf16.reshape(E * H, I), mode)
        self.q1 = (c1, s1, self.g1)
        self.q2 = (c2, s2, self.g2)
        self.d1 = dequantize(c1, s1)
        self.d2 = dequantize(c2, s2)


def moe_forward(x_bf16, ids, probs, weights: DequantWeights, mode: int = SCALE_RU, intermediates: bool = False):
    """The layer (miniTE page, "how it differs" / "how to use it"; article 4.4-4.5).

    x [T,H] BF16 bits, ids/probs [T,K].  Returns out [T,H] BF16 bits, and with
    ``intermediates`` also per-pair y1 [P,2I], h [P,I], amax2 [P], y2 [P,H]."""
    x = _c(x_bf16, np.uint16)
    ids = _c(ids, np.int32)
    probs = _c(probs, np.float32)
    T, H = x.shape
    K = ids.shape[1]
    I = weights.I
    assert H == weights.H
    if ids.size and (ids.min() < 0 or ids.max() >= weights.E):
        raise ValueError("expert id out of range")
    P = T * K
    out = np.empty((T, H), np.uint16)
    y1 = np.empty((P, 2 * I), np.uint16) if intermediates else None
    h = np.empty((P, I), np.uint16) if intermediates else None
    amax2 = np.empty((P,), np.float32) if intermediates else None
    y2 = np.empty((P, H), np.uint16) if intermediates else None
    _load().orc_moe_forward_deq(_p(x), T, H, I, K, _p(ids), _p(probs), _p(weights.d1), _p(weights.g1),
                                _p(weights.d2), _p(weights.g2), int(mode), _p(out), _p(y1), _p(h), _p(amax2),
                                _p(y2))
    if intermediates:
        return out, dict(y1=y1, h=h, amax2=amax2, y2=y2)
    return out
