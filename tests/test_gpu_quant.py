"""GPU quantizer parity: nvfp4_quantize and nvfp4moe_quantize_weights through
the C ABI, bit-exact against the CPU oracle (codes, scales and g), in both
layouts and both scale roundings (miniTE summary page, "how it differs")."""
import json
import os
import struct

import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import code_tie_rows, gemm_to_logical, scale_tie_rows, scale_tie_targets, to_dev, to_host, unpack_codes

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_hand_cases.json")


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_moe_expert_sort_amd as m
    m.lib()  # raises if the HIP library is missing
    return m, torch.device("cuda:0")


def _gpu_quant(m, dev, x_bits, mode, layout, ld=None):
    import torch
    rows, cols = x_bits.shape
    if ld is None or ld == cols:
        xd = to_dev(x_bits, dev)
    else:
        pad = np.zeros((rows, ld), np.uint16)
        pad[:, :cols] = x_bits
        xd = to_dev(pad, dev)[:, :cols]
    codes, scales, g = m.quantize(xd, layout=layout, scale_round=mode)
    torch.cuda.synchronize()
    c, s, gg = to_host(codes), to_host(scales), to_host(g)
    if layout == m.LAYOUT_GEMM:
        c, s = gemm_to_logical(c, s, rows, cols)
    return c, s, gg


def _assert_same(got, want, what):
    c, s, g = got
    wc, ws, wg = want
    assert np.array_equal(s, ws), f"{what}: scales differ at {np.argwhere(s != ws)[:5].tolist()}"
    assert np.array_equal(c, wc), f"{what}: codes differ at {np.argwhere(c != wc)[:5].tolist()}"
    assert np.array_equal(g.view(np.uint32), wg.view(np.uint32)), f"{what}: g differs"


def _rows(seed, rows, cols):
    rng = np.random.default_rng(seed)
    parts = [rng.standard_normal((rows, cols))]
    x = rng.standard_normal((rows, cols))
    x[rng.random((rows, cols)) < 0.01] *= 50
    parts.append(x)
    parts.append(rng.standard_normal((rows, cols)) * 10.0 ** rng.integers(-30, 30, (rows, 1)))
    y = rng.standard_normal((rows, cols))
    y *= 10.0 ** rng.integers(-9, 1, (rows, cols // 16)).repeat(16, axis=1)
    parts.append(y)
    z = rng.standard_normal((rows, cols))
    z[rng.random((rows, cols)) < 0.7] = 0.0
    parts.append(z)
    out = W.f32_to_bf16_bits(np.concatenate(parts).astype(np.float32))
    out[1] = 0                 # zero row
    out[2, ::3] = 0x8000       # negative zeros
    out[3, :] = 0x8000         # all negative zero
    return out


def test_hand_cases(gpu, orc):
    m, dev = gpu
    cases = json.load(open(GOLDEN))["cases"]
    for case in cases:
        vals = [struct.unpack("<I", struct.pack("<f", float(v)))[0] >> 16 for v in case["x"]]
        x = np.array([vals], np.uint16)
        for mode, key in ((0, "ru"), (1, "rne")):
            c, s, g = _gpu_quant(m, dev, x, mode, m.LAYOUT_LOGICAL)
            want = case[key]
            assert [int(v) for v in c[0]] == [int(v, 16) for v in want["codes"]], (case["name"], key)
            assert [int(v) for v in s[0]] == [int(v, 16) for v in want["scales"]], (case["name"], key)
            assert int(g.view(np.uint32)[0]) == int(want["g"], 16), (case["name"], key)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("cols", [16, 32, 128, 256, 512, 768, 1024, 1056, 2048])
def test_random_rows_logical(gpu, orc, mode, cols):
    # Rows of at most 1024 columns go 8, 4 or 2 to a wavefront (up to 256, 512
    # and 1024 columns); 1056 is the shortest row with a wavefront of its own.
    m, dev = gpu
    x = _rows(100 + cols, 13, cols)  # 65 rows: no multiple of the rows per block in any path
    _assert_same(_gpu_quant(m, dev, x, mode, m.LAYOUT_LOGICAL), orc.quantize(x, mode), f"cols={cols} mode={mode}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("cols", [128, 512, 768, 1024, 2048])
def test_random_rows_gemm_layout(gpu, orc, mode, cols):
    m, dev = gpu
    x = _rows(200 + cols, 32, cols)[:160]
    _assert_same(_gpu_quant(m, dev, x, mode, m.LAYOUT_GEMM), orc.quantize(x, mode), f"gemm cols={cols}")


def test_strided_rows(gpu, orc):
    m, dev = gpu
    x = _rows(7, 4, 256)
    _assert_same(_gpu_quant(m, dev, x, 0, m.LAYOUT_LOGICAL, ld=264), orc.quantize(x, 0), "ld=264")


def test_dense_workload_inputs_bit_exact(gpu, orc):
    """X with 1% outliers x50 [4096, 2048] and W [1536, 2048] of the dense linear workload."""
    m, dev = gpu
    wl = W.dense(seed=1)
    _assert_same(_gpu_quant(m, dev, wl.x, 0, m.LAYOUT_GEMM), orc.quantize(wl.x, 0), "dense X")
    _assert_same(_gpu_quant(m, dev, wl.w, 0, m.LAYOUT_GEMM), orc.quantize(wl.w, 0), "dense W")
    _assert_same(_gpu_quant(m, dev, wl.x, 1, m.LAYOUT_LOGICAL), orc.quantize(wl.x, 1), "dense X rne")


@pytest.mark.parametrize("mode", [0, 1])
def test_quantize_weights_tiny_layer(gpu, orc, mode):
    import torch
    m, dev = gpu
    wl = W.tiny(seed=0)
    s = wl.shape
    w1, w2 = wl.weights(threads=4)
    cfg = m.make_config(s.H, s.I, s.E, s.K, s.T, scale_round=mode)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    torch.cuda.synchronize()
    c1, s1 = gemm_to_logical(to_host(qw.w1_codes), to_host(qw.w1_scales), s.E * 2 * s.I, s.H)
    c2, s2 = gemm_to_logical(to_host(qw.w2_codes), to_host(qw.w2_scales), s.E * s.H, s.I)
    _assert_same((c1, s1, to_host(qw.w1_g)), orc.quantize(w1.reshape(-1, s.H), mode), "W1")
    _assert_same((c2, s2, to_host(qw.w2_g)), orc.quantize(w2.reshape(-1, s.I), mode), "W2")


def test_quantize_weights_qwen3_experts(gpu, orc):
    """Full Qwen3-30B-A3B-shaped expert weights; every expert checked bit-exact."""
    import torch
    m, dev = gpu
    wl = W.qwen3(seed=2, T=8)
    s = wl.shape
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, 8)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    torch.cuda.synchronize()
    c1, s1 = gemm_to_logical(to_host(qw.w1_codes), to_host(qw.w1_scales), s.E * 2 * s.I, s.H)
    _assert_same((c1, s1, to_host(qw.w1_g)), orc.quantize(w1.reshape(-1, s.H), 0), "W1 qwen3")
    c2, s2 = gemm_to_logical(to_host(qw.w2_codes), to_host(qw.w2_scales), s.E * s.H, s.I)
    _assert_same((c2, s2, to_host(qw.w2_g)), orc.quantize(w2.reshape(-1, s.I), 0), "W2 qwen3")


def test_scale_encoder_ties(gpu, orc):
    """The E4M3 block-scale encoder at every decision point, both roundings and
    layouts: scales equal the format's expectation, codes, scales and g equal
    the oracle bit for bit."""
    m, dev = gpu
    x, want = scale_tie_rows(rows_multiple=32)  # whole 32-row tiles for the GEMM layout
    for mode in (0, 1):
        ref = orc.quantize(x, mode)
        assert np.array_equal(ref[1], want[mode]), f"oracle scales vs the format, mode {mode}"
        for layout in (m.LAYOUT_LOGICAL, m.LAYOUT_GEMM):
            got = _gpu_quant(m, dev, x, mode, layout)
            assert np.array_equal(got[1], want[mode]), f"GPU scales vs the format, mode {mode} layout {layout}"
            _assert_same(got, ref, f"scale ties mode={mode} layout={layout}")
    print(f"  {len(scale_tie_targets())} block maxima at the E4M3 decision points, both roundings, both layouts")


def test_code_decisions_at_every_scale(gpu, orc):
    """E2M1 element codes at every decision point under each of the 126 E4M3
    scales (quotients landing exactly on a threshold or a BF16 step beside
    it, both signs): GPU equal to the format's expectation and to the oracle
    bit for bit, both roundings and layouts."""
    m, dev = gpu
    x, want = code_tie_rows()
    for mode in (0, 1):
        ref = orc.quantize(x, mode)
        for layout in (m.LAYOUT_LOGICAL, m.LAYOUT_GEMM):
            got = _gpu_quant(m, dev, x, mode, layout)
            assert np.array_equal(unpack_codes(got[0]), want), f"GPU codes vs the format, mode {mode} layout {layout}"
            _assert_same(got, ref, f"code ties mode={mode} layout={layout}")
