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
