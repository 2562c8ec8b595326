"""Shared test helpers: device transfer, the GEMM-layout map written from the
header's documentation, error metrics.  Imports neither the oracle nor the
HIP package by itself."""
from __future__ import annotations

import numpy as np

import moe_workloads as W


def to_dev(a: np.ndarray, dev):
    import torch
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a


def gemm_layout_maps(rows: int, cols: int):
    """Index maps GEMM layout -> logical, from include/nvfp4moe.h:
    code byte  = (rt*(cols/64) + c)*1024 + (h*32 + rl)*16 + (k%32)/2
    scale byte = (rt*(cols/128) + c/2)*256 + (h*32 + rl)*4 + (c%2)*2 + (k%32)/16
    Returns (code_src [rows, cols/2], scale_src [rows, cols/16]) flat GEMM offsets
    of each logical byte (logical code byte i of row r holds columns 2i, 2i+1)."""
    r = np.arange(rows)[:, None]
    rt, rl = r // 32, r % 32
    k = np.arange(0, cols, 2)[None, :]
    c, h = k // 64, (k // 32) % 2
    code_src = (rt * (cols // 64) + c) * 1024 + (h * 32 + rl) * 16 + (k % 32) // 2
    kb = np.arange(0, cols, 16)[None, :]
    c, h = kb // 64, (kb // 32) % 2
    scale_src = (rt * (cols // 128) + c // 2) * 256 + (h * 32 + rl) * 4 + (c % 2) * 2 + (kb % 32) // 16
    return code_src, scale_src


def gemm_to_logical(codes_flat: np.ndarray, scales_flat: np.ndarray, rows: int, cols: int):
    cs, ss = gemm_layout_maps(rows, cols)
    return codes_flat.reshape(-1)[cs], scales_flat.reshape(-1)[ss]


def rel_l2(got_bits: np.ndarray, ref_bits: np.ndarray):
    g = W.bf16_bits_to_f32(got_bits).astype(np.float64)
    r = W.bf16_bits_to_f32(ref_bits).astype(np.float64)
    den = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / (den if den > 0 else 1.0)
    return rel, float(np.abs(g - r).max()) if g.size else 0.0


def bf16(a) -> np.ndarray:
    return W.f32_to_bf16_bits(np.asarray(a, np.float32))


def e4m3fn_value(code: int) -> float:
    """E4M3FN value of a positive code (1..126), from the format: bias 7,
    three mantissa bits, subnormals m * 2^-9."""
    e, mant = code >> 3, code & 7
    return mant * 2.0 ** -9 if e == 0 else 2.0 ** (e - 7) * (1.0 + mant / 8.0)


def bf16_exact_bits(v: float) -> int:
    b = int(W.f32_to_bf16_bits(np.array([v], np.float32))[0])
    assert W.bf16_bits_to_f32(np.array([b], np.uint16))[0] == np.float32(v), v  # exactly representable
    return b


def scale_tie_targets():
    """(BF16 bits of a block maximum, expected RU scale code, expected RNE scale code).

    With the row maximum 448, fl32(6 * fl32(448 / 2688)) is exactly 1.0, so a
    block's scale input v = amax_b / (6 g) equals its maximum: every E4M3FN
    value, every midpoint between neighbours (ties: RU takes the upper code,
    RNE the one with the even mantissa, i.e. the even code) and the BF16
    values either side of each midpoint land on the encoder's decisions."""
    out = []
    for c in range(1, 127):
        out.append((bf16_exact_bits(e4m3fn_value(c)), c, c))
    lo_mid = bf16_exact_bits(2.0 ** -10)  # between 0 and the smallest subnormal 2^-9
    out += [(lo_mid, 1, 0), (lo_mid - 1, 1, 0), (lo_mid + 1, 1, 1)]
    for c in range(1, 126):
        mid = bf16_exact_bits((e4m3fn_value(c) + e4m3fn_value(c + 1)) / 2)
        even = c if c % 2 == 0 else c + 1
        out += [(mid, c + 1, even), (mid - 1, c + 1, c), (mid + 1, c + 1, c + 1)]
    return out



def scale_tie_rows(rows_multiple: int = 1):
    """BF16 rows of 128 columns holding every scale_tie_targets() block maximum:
    block 0 of each row pins the row maximum at 448 (so 6 g = 1 exactly),
    blocks 1..7 take one target each; the block's other elements are fixed
    fractions of its maximum.  Returns (rows, {mode: expected scale codes})."""
    targets = scale_tie_targets()
    pattern = np.array([1, -0.75, 0.5, 0.3, -0.2, 0.1, 0.05, -0.9, 0.6, 0.4, -0.33, 0.25, 0.125, -0.01, 0.7, 0.0])
    per_row = 7
    n_rows = (len(targets) + per_row - 1) // per_row
    n_rows = (n_rows + rows_multiple - 1) // rows_multiple * rows_multiple
    x = np.zeros((n_rows, 128), np.uint16)
    want = {0: np.zeros((n_rows, 8), np.uint8), 1: np.zeros((n_rows, 8), np.uint8)}
    for r in range(n_rows):
        x[r, :16] = W.f32_to_bf16_bits((448.0 * pattern).astype(np.float32))
        want[0][r, 0] = want[1][r, 0] = 0x7E
    for i, (bits, ru, rne) in enumerate(targets):
        r, b = divmod(i, per_row)
        t = float(W.bf16_bits_to_f32(np.array([bits], np.uint16))[0])
        blk = W.f32_to_bf16_bits((t * pattern).astype(np.float32))
        blk[0] = bits  # the block maximum is exactly the target
        assert np.all((blk & 0x7FFF) <= bits)
        x[r, 16 * (b + 1):16 * (b + 2)] = blk
        want[0][r, b + 1], want[1][r, b + 1] = ru, rne
    return x, want  # blocks without a target stay zero (scale 0)


# E2M1 decision thresholds (midpoints between neighbouring magnitudes) and the
# code each tie rounds to (the even code), with the codes on either side.
E2M1_TIES = ((0.25, 0, 0, 1), (0.75, 2, 1, 2), (1.25, 2, 2, 3), (1.75, 4, 3, 4), (2.5, 4, 4, 5), (3.5, 6, 5, 6),
             (5.0, 6, 6, 7))


def code_tie_rows():
    """BF16 rows of 128 columns and their expected E2M1 codes (both scale
    roundings give the same here).  Block 0 of each row holds the row maximum
    2688, so g = 1 exactly; every other block has maximum 6 S for an E4M3FN
    value S, so its scale is exactly S, and its remaining elements are
    theta * S for each E2M1 decision threshold theta, and the BF16 values
    either side, with both signs: the quotient x / S lands on the threshold
    or just beside it.  Returns (rows, expected codes [rows, 128] uint8)."""
    blocks = []  # list of (S, [(bf16 bits, code)] with 16 entries)
    for c in range(1, 127):
        S = e4m3fn_value(c)
        items = []
        for theta, tie, below, above in E2M1_TIES:
            b = bf16_exact_bits(theta * S)
            for bits, code in ((b, tie), (b - 1, below), (b + 1, above)):
                for sign in (0, 0x8000):
                    items.append((bits | sign, code | (8 if sign else 0)))
        top = bf16_exact_bits(6 * S)
        for k in range(0, len(items), 15):
            chunk = items[k:k + 15]
            chunk += [(0, 0)] * (15 - len(chunk))
            blocks.append([(top, 7)] + chunk)
    per_row = 7
    n_rows = (len(blocks) + per_row - 1) // per_row
    n_rows = (n_rows + 31) // 32 * 32
    x = np.zeros((n_rows, 128), np.uint16)
    codes = np.zeros((n_rows, 128), np.uint8)
    for r in range(n_rows):
        x[r, 0] = bf16_exact_bits(2688.0)
        codes[r, 0] = 7  # 2688 / (448 * 1) = 6; the rest of block 0 is zero
    for i, blk in enumerate(blocks):
        r, b = divmod(i, per_row)
        for j, (bits, code) in enumerate(blk):
            x[r, 16 * (b + 1) + j] = bits
            codes[r, 16 * (b + 1) + j] = code
    return x, codes


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[rows, cols/2] packed E2M1 bytes (element 2i in the low nibble) -> [rows, cols] codes."""
    out = np.empty((packed.shape[0], packed.shape[1] * 2), np.uint8)
    out[:, 0::2] = packed & 0xF
    out[:, 1::2] = packed >> 4
    return out
