"""The forward with the activations' max, quantization and FC1 GEMM fused
(miniTE summary page, "assumptions and limits": the online
amax-quantization-GEMM fusion, whose numerical validation the page leaves
open) against the standard forward, through the C ABI.

The online forward never builds the sorted, quantized copy of X: the sort
records each token's max |x| and FC1 quantizes each sorted row's BF16 token
row itself.  Every quantized group must come out as the standard quantizer
made it, so FC1's output h (with its per-32-column maxima), FC2's input and
output and the layer output must be the standard forward's bit for bit --
on the tiny layer in both scale roundings, odd shapes (K = E, a partial
column tile, one expert, token rows of 4224 and 8320 columns, which the
sort's max takes in registers and in its wave loop), the Qwen3-shaped layer
at T = 4096 and Zipf-skewed
routing at T = 16384 -- and the standard forward is itself compared element
by element with the oracle (tests/test_gpu_layer.py).  Each token's output
is also bitwise the same alone as in its batch."""
import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_moe_expert_sort_amd as m
    m.lib()
    return m, torch.device("cuda:0")


def _compare(m, dev, wl, mode=0, T=None):
    import torch
    s = wl.shape
    T = s.T if T is None else T
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, s.T, scale_round=mode)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    x, ids, probs = to_dev(wl.x[:T], dev), to_dev(wl.ids[:T], dev), to_dev(wl.probs[:T], dev)
    ws_a, ws_b = m.alloc_workspace(cfg, dev), m.alloc_workspace(cfg, dev)
    ws_b.fill_(0xA5)  # stale contents must not leak into the online forward's results
    ref = m.moe_expert_forward(cfg, x, ids, probs, qw, ws_a)
    got = m.moe_expert_forward_online(cfg, x, ids, probs, qw, ws_b)
    torch.cuda.synchronize()
    assert m.device_error(cfg, ws_a) == 0 and m.device_error(cfg, ws_b) == 0
    lay = m.workspace_layout(cfg)

    def view(ws, off, dtype, count):
        return ws[off:off + count * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    rows = int(to_host(view(ws_a, lay.expert_off, torch.int32, s.E + 1))[-1])
    for name, off in (("row2pair", lay.row2pair), ("expert_off", lay.expert_off)):
        n = rows if name == "row2pair" else s.E + 1
        assert torch.equal(view(ws_a, off, torch.int32, n), view(ws_b, off, torch.int32, n)), name
    valid = view(ws_a, lay.row2pair, torch.int32, rows) >= 0
    for name, off, width, dtype in (("h", lay.h, s.I, torch.int16), ("FC2 output y2", lay.y2, s.H, torch.int16),
                                    ("A2 codes", lay.a2_codes, s.I // 2, torch.uint8),
                                    ("max |h| per 32 columns", lay.amax2_part, s.I // 32, torch.int32)):
        a = view(ws_a, off, dtype, rows * width).view(rows, width)[valid]
        b = view(ws_b, off, dtype, rows * width).view(rows, width)[valid]
        assert torch.equal(a, b), name
    assert torch.equal(ref.view(torch.int16), got.view(torch.int16)), "layer output"
    return cfg, qw, got


@pytest.mark.parametrize("mode", [0, 1])
def test_online_equals_standard_tiny(gpu, mode):
    m, dev = gpu
    _compare(m, dev, W.tiny(seed=0), mode)


@pytest.mark.parametrize("shape", [W.MoEShape(T=37, H=384, E=5, K=5, I=384),    # every token to every expert
                                   W.MoEShape(T=450, H=256, E=3, K=2, I=640),   # a partial FC1 column tile
                                   W.MoEShape(T=200, H=128, E=1, K=1, I=128),   # one expert
                                   W.MoEShape(T=40, H=4224, E=4, K=2, I=128),    # 3 register groups per lane
                                   W.MoEShape(T=24, H=8320, E=3, K=2, I=128)])   # the sort's wave loop
def test_online_equals_standard_odd_shapes(gpu, shape):
    m, dev = gpu
    _compare(m, dev, W.MoEWorkload("odd", 12, shape))


def test_online_equals_standard_qwen3(gpu):
    m, dev = gpu
    _compare(m, dev, W.qwen3(seed=2))


def test_online_equals_standard_skewed(gpu):
    m, dev = gpu
    _compare(m, dev, W.skewed(seed=3))


def test_online_batch_invariance(gpu):
    """Tokens alone (T = 1, 3, 17) give the bits they get in the 4096-token batch."""
    import torch
    m, dev = gpu
    wl = W.qwen3(seed=2)
    cfg, qw, full = _compare(m, dev, wl)
    full = to_host(full)
    ws = m.alloc_workspace(cfg, dev)
    for T in (1, 3, 17):
        out = m.moe_expert_forward_online(cfg, to_dev(wl.x[:T], dev), to_dev(wl.ids[:T], dev),
                                          to_dev(wl.probs[:T], dev), qw, ws)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out).view(np.uint16), full[:T].view(np.uint16)), f"T={T}"
