"""Fused vs unfused pipeline, bit for bit (the miniTE page, "assumptions and
limits": the fused path is checked bitwise against the unfused quantization
and GEMM API; "how to use it": the prior order was sort, pad(X), amax scan,
quantize, which the fused path replaces by sort+amax, pad, quantize).

The unfused path is built from the library's own public entry points, one
separate launch per step:
  sort      the forward's row2pair (itself checked against the oracle's sort
            in test_gpu_layer.py);
  pad(X)    a BF16 matrix with each sorted row's token row and zero padding rows;
  amax+quant nvfp4_quantize on that matrix (GEMM layout), which scans each
            row's amax itself;
  FC2       nvfp4_linear per expert on that expert's rows of h with the
            expert's W2.
It must reproduce the fused forward's A1 (sorted, padded, quantized X), A2
(quantized h, whose amax came from the SwiGLU producer) and y2 bit for bit.

FC1 and the producer: the library's unfused forward runs FC1 as a plain
grouped GEMM writing y1 (both halves, gate and up) and then the router-
weighted SwiGLU producer as a kernel of its own; its h, the per-32-column
maxima of |h|, A2, y2 and the output must be the fused forward's bit for bit
(the fused FC1 epilogue forms the same y1 values in registers)."""
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


def _fused_vs_unfused(m, dev, wl, mode):
    import torch
    s = wl.shape
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, s.T, scale_round=mode)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    ws = m.alloc_workspace(cfg, dev)
    lay = m.workspace_layout(cfg)
    x = to_dev(wl.x, dev)
    m.moe_expert_forward(cfg, x, to_dev(wl.ids, dev), to_dev(wl.probs, dev), qw, ws)
    torch.cuda.synchronize()
    assert m.device_error(cfg, ws) == 0

    def view(off, dtype, count):
        return ws[off:off + count * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    off = to_host(view(lay.expert_off, torch.int32, s.E + 1)).astype(np.int64)
    cnt = to_host(view(lay.expert_count, torch.int32, s.E)).astype(np.int64)
    rows = int(off[-1])
    r2p = view(lay.row2pair, torch.int32, rows).long()
    valid = r2p >= 0
    tok = torch.where(valid, r2p // s.K, torch.zeros_like(r2p))

    # A1: sort -> pad(X) -> amax scan + quantize, as separate steps
    xs = torch.where(valid[:, None], x.view(torch.int16)[tok], torch.zeros((), dtype=torch.int16, device=dev))
    c, sc, g = m.quantize(xs.contiguous(), layout=m.LAYOUT_GEMM, scale_round=mode)
    assert torch.equal(view(lay.a1_codes, torch.uint8, rows * s.H // 2), c.view(-1)), "A1 codes"
    assert torch.equal(view(lay.a1_scales, torch.uint8, rows * s.H // 16), sc.view(-1)), "A1 scales"
    assert torch.equal(view(lay.a1_g, torch.int32, rows), g.view(torch.int32)), "A1 g"

    # A2: h -> amax scan + quantize (padding rows of h are never written: zero them)
    h = view(lay.h, torch.int16, rows * s.I).view(rows, s.I)
    hz = torch.where(valid[:, None], h, torch.zeros((), dtype=torch.int16, device=dev)).contiguous()
    c2, sc2, g2 = m.quantize(hz, layout=m.LAYOUT_GEMM, scale_round=mode)
    assert torch.equal(view(lay.a2_codes, torch.uint8, rows * s.I // 2), c2.view(-1)), "A2 codes"
    assert torch.equal(view(lay.a2_scales, torch.uint8, rows * s.I // 16), sc2.view(-1)), "A2 scales"
    assert torch.equal(view(lay.a2_g, torch.int32, rows), g2.view(torch.int32)), "A2 g"

    # FC2: the dense GEMM entry point per expert on that expert's rows
    y2 = view(lay.y2, torch.int16, rows * s.H).view(rows, s.H)
    lws = torch.empty((m.linear_workspace_bytes(int(cnt.max()), s.I),), dtype=torch.uint8, device=dev)
    checked = 0
    for e in range(s.E):
        if cnt[e] == 0:
            continue
        r0, n = int(off[e]), int(cnt[e])
        We = m.qtensor(qw.w2_codes[e * s.H:(e + 1) * s.H], qw.w2_scales[e * s.H:(e + 1) * s.H],
                       qw.w2_g[e * s.H:(e + 1) * s.H], 1, s.H, s.I)
        ye = m.linear(h[r0:r0 + n], We, lws, scale_round=mode)
        assert torch.equal(ye, y2[r0:r0 + n]), f"y2 rows of expert {e}"
        checked += n
    torch.cuda.synchronize()
    assert checked == s.T * s.K
    print(f"  fused == unfused: A1 and A2 over {rows} rows, y2 over {checked} rows in {int((cnt > 0).sum())} experts")


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_equals_unfused_tiny(gpu, mode):
    m, dev = gpu
    _fused_vs_unfused(m, dev, W.tiny(seed=0), mode)


def test_fused_equals_unfused_qwen3(gpu):
    m, dev = gpu
    _fused_vs_unfused(m, dev, W.qwen3(seed=2, T=4096), 0)


def test_fused_equals_unfused_skewed(gpu):
    m, dev = gpu
    _fused_vs_unfused(m, dev, W.skewed(seed=3), 0)


def _fused_vs_unfused_fc1(m, dev, wl, mode):
    import torch
    s = wl.shape
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, s.T, scale_round=mode)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    lay = m.workspace_layout(cfg)
    x, ids, probs = to_dev(wl.x, dev), to_dev(wl.ids, dev), to_dev(wl.probs, dev)
    ws_f, ws_u = m.alloc_workspace(cfg, dev), m.alloc_workspace(cfg, dev)
    out_f = m.moe_expert_forward(cfg, x, ids, probs, qw, ws_f)
    out_u, y1 = m.moe_expert_forward_unfused(cfg, x, ids, probs, qw, ws_u)
    torch.cuda.synchronize()
    assert m.device_error(cfg, ws_f) == 0 and m.device_error(cfg, ws_u) == 0

    def view(ws, off, dtype, count):
        return ws[off:off + count * torch.tensor([], dtype=dtype).element_size()].view(dtype)

    rows = int(to_host(view(ws_f, lay.expert_off, torch.int32, s.E + 1))[-1])
    valid = view(ws_f, lay.row2pair, torch.int32, rows) >= 0
    for name, n in (("h", s.I), ("y2", s.H)):
        a = view(ws_f, getattr(lay, name), torch.int16, rows * n).view(rows, n)[valid]
        b = view(ws_u, getattr(lay, name), torch.int16, rows * n).view(rows, n)[valid]
        assert torch.equal(a, b), name
    a = view(ws_f, lay.amax2_part, torch.int32, rows * lay.n_part).view(rows, lay.n_part)[valid]
    b = view(ws_u, lay.amax2_part, torch.int32, rows * lay.n_part).view(rows, lay.n_part)[valid]
    assert torch.equal(a, b), "FC2 maxima from the producer"
    for name, n in (("a2_codes", s.I // 2), ("a2_scales", s.I // 16), ("a2_g", 4)):
        assert torch.equal(view(ws_f, getattr(lay, name), torch.uint8, rows * n),
                           view(ws_u, getattr(lay, name), torch.uint8, rows * n)), name
    assert torch.equal(out_f, out_u), "outputs"
    print(f"  fused FC1 + producer == unfused over {int(valid.sum())} rows: h, maxima, A2, y2, out")


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_fc1_producer_equals_unfused_tiny(gpu, mode):
    m, dev = gpu
    _fused_vs_unfused_fc1(m, dev, W.tiny(seed=0), mode)


def test_fused_fc1_producer_equals_unfused_qwen3(gpu):
    m, dev = gpu
    _fused_vs_unfused_fc1(m, dev, W.qwen3(seed=2, T=4096), 0)


def test_fused_fc1_producer_equals_unfused_skewed(gpu):
    m, dev = gpu
    _fused_vs_unfused_fc1(m, dev, W.skewed(seed=3), 0)
