"""GPU parity of the NVFP4 MoE expert forward and the dense NVFP4 linear,
through the C ABI, against the CPU oracle.

Bars: integer/byte work (expert sort, device offsets, quantized buffers, the
FC2 amax, the combine given the GPU's expert outputs) bit-exact; BF16 layer
outputs within relative L2 <= 1e-2 of the oracle (max-abs reported).
Sources: miniTE summary page, "how it differs" and "how to use it"; article
sections 4.4 and 4.5."""
import ctypes

import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import gemm_to_logical, rel_l2, to_dev, to_host

pytestmark = pytest.mark.gpu

REL_L2_TOL = 1e-2


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_moe_expert_sort_amd as m
    m.lib()
    return m, torch.device("cuda:0")


class Layer:
    """A workload's weights quantized on the GPU plus a workspace for max_tokens."""

    def __init__(self, m, dev, wl, max_tokens, mode=0, weights=None):
        import torch
        s = wl.shape
        self.m, self.dev, self.wl, self.s = m, dev, wl, s
        self.w1, self.w2 = weights if weights is not None else wl.weights(threads=16)
        self.cfg = m.make_config(s.H, s.I, s.E, s.K, max_tokens, scale_round=mode)
        self.qw = m.QuantWeights(self.cfg, dev).quantize_from(to_dev(self.w1, dev), to_dev(self.w2, dev))
        self.ws = m.alloc_workspace(self.cfg, dev)
        self.lay = m.workspace_layout(self.cfg)
        torch.cuda.synchronize()

    def forward(self, x, ids, probs):
        import torch
        out = self.m.moe_expert_forward(self.cfg, to_dev(x, self.dev), to_dev(ids, self.dev),
                                        to_dev(probs, self.dev), self.qw, self.ws)
        torch.cuda.synchronize()
        return to_host(out)

    def ws_array(self, off, dtype, count):
        a = to_host(self.ws[off:off + count * np.dtype(dtype).itemsize])
        return a.view(dtype)


def _oracle_subset(orc, layer, x, ids, probs, mode=0, intermediates=False):
    """Oracle forward on a token subset, with only the experts those tokens use."""
    used = np.unique(ids)
    remap = np.full(layer.s.E, -1, np.int32)
    remap[used] = np.arange(used.size)
    wts = orc.DequantWeights(layer.w1[used], layer.w2[used], mode)
    return orc.moe_forward(x, remap[ids], probs, wts, mode, intermediates=intermediates)


def _check_route(orc, layer, ids, T):
    s = layer.s
    off, pair2row, row2pair = orc.route(ids, s.E, 32)
    lay = layer.lay
    got_off = layer.ws_array(lay.expert_off, np.int32, s.E + 1)
    got_cnt = layer.ws_array(lay.expert_count, np.int32, s.E)
    got_p2r = layer.ws_array(lay.pair2row, np.int32, T * s.K)
    got_r2p = layer.ws_array(lay.row2pair, np.int32, int(off[-1]))
    assert np.array_equal(got_off, off), "expert offsets"
    assert np.array_equal(got_cnt, np.bincount(ids.reshape(-1), minlength=s.E)), "expert counts"
    assert np.array_equal(got_p2r, pair2row), "pair -> sorted row"
    assert np.array_equal(got_r2p, row2pair), "sorted row -> pair"
    return off, pair2row


def _check_a1(orc, layer, x, pair2row, mode):
    """The padded, sorted, quantized X buffer equals the oracle's Q of each token, per copy."""
    s, lay = layer.s, layer.lay
    rows = int(lay.rows_cap)
    c = layer.ws_array(lay.a1_codes, np.uint8, rows * s.H // 2)
    sc = layer.ws_array(lay.a1_scales, np.uint8, rows * s.H // 16)
    g = layer.ws_array(lay.a1_g, np.float32, rows)
    lc, ls = gemm_to_logical(c, sc, rows, s.H)
    wc, wsc, wg = orc.quantize(x, mode)
    tok = np.arange(pair2row.size) // s.K
    assert np.array_equal(lc[pair2row], wc[tok]), "A1 codes"
    assert np.array_equal(ls[pair2row], wsc[tok]), "A1 scales"
    assert np.array_equal(g[pair2row].view(np.uint32), wg[tok].view(np.uint32)), "A1 g"


def _stage_checks(orc, layer, x, ids, probs, out, mode):
    """Per-stage parity on a small workload: sort, A1, h, FC2 amax, A2, y2, combine."""
    s, lay = layer.s, layer.lay
    T = x.shape[0]
    P = T * s.K
    off, pair2row = _check_route(orc, layer, ids, T)
    _check_a1(orc, layer, x, pair2row, mode)
    ref_out, mid = _oracle_subset(orc, layer, x, ids, probs, mode, intermediates=True)
    rows = int(lay.rows_cap)
    h = layer.ws_array(lay.h, np.uint16, rows * s.I).reshape(rows, s.I)[pair2row]
    rel_h, mx_h = rel_l2(h, mid["h"])
    assert rel_h <= REL_L2_TOL, f"h rel L2 {rel_h}"
    # the producer's maxima are those of the BF16 tensor FC2 consumes
    part = layer.ws_array(lay.amax2_part, np.float32, rows * lay.n_part).reshape(rows, lay.n_part)[pair2row]
    hv = np.abs(W.bf16_bits_to_f32(h))
    assert np.array_equal(part.max(axis=1), hv.max(axis=1)), "FC2 amax from the producer"
    for j in range(lay.n_part):
        assert np.array_equal(part[:, j], hv[:, 32 * j:32 * (j + 1)].max(axis=1)), f"column group {j} max"
    # A2 = Q(h) bit-exact, given the GPU's own h
    c = layer.ws_array(lay.a2_codes, np.uint8, rows * s.I // 2)
    sc = layer.ws_array(lay.a2_scales, np.uint8, rows * s.I // 16)
    g = layer.ws_array(lay.a2_g, np.float32, rows)
    lc, ls = gemm_to_logical(c, sc, rows, s.I)
    wc, wsc, wg = orc.quantize(h, mode)
    assert np.array_equal(lc[pair2row], wc) and np.array_equal(ls[pair2row], wsc), "A2 = Q(h)"
    assert np.array_equal(g[pair2row].view(np.uint32), wg.view(np.uint32)), "A2 g"
    # y2 within tolerance; the combine bit-exact on the GPU's own y2
    y2 = layer.ws_array(lay.y2, np.uint16, rows * s.H).reshape(rows, s.H)[pair2row]
    rel_y2, _ = rel_l2(y2, mid["y2"])
    assert rel_y2 <= REL_L2_TOL, f"y2 rel L2 {rel_y2}"
    assert np.array_equal(orc.combine(y2.reshape(T, s.K, s.H)), out), "combine of the GPU's y2"
    rel, mx = rel_l2(out, ref_out)
    print(f"  stages: h rel {rel_h:.2e}, y2 rel {rel_y2:.2e}, out rel {rel:.2e} max-abs {mx:.3e}")
    assert rel <= REL_L2_TOL, f"out rel L2 {rel}"


@pytest.mark.parametrize("mode", [0, 1])
def test_tiny_layer_all_stages(gpu, orc, mode):
    m, dev = gpu
    wl = W.tiny(seed=0)
    layer = Layer(m, dev, wl, max_tokens=wl.shape.T, mode=mode)
    out = layer.forward(wl.x, wl.ids, wl.probs)
    _stage_checks(orc, layer, wl.x, wl.ids, wl.probs, out, mode)
    assert m.device_error(layer.cfg, layer.ws) == 0


def test_tiny_layer_ragged_batches(gpu, orc):
    """Token counts that leave partial tiles everywhere: 1, 3, 17, 33, 64."""
    m, dev = gpu
    wl = W.tiny(seed=5)
    layer = Layer(m, dev, wl, max_tokens=64)
    for T in (1, 3, 17, 33, 64):
        out = layer.forward(wl.x[:T], wl.ids[:T], wl.probs[:T])
        _stage_checks(orc, layer, wl.x[:T], wl.ids[:T], wl.probs[:T], out, 0)


def test_routing_edge_cases(gpu, orc):
    """Every token to the same experts; experts with no tokens; K = 1."""
    m, dev = gpu
    shape = W.MoEShape(T=40, H=256, E=8, K=2, I=128)
    wl = W.MoEWorkload("edge", 9, shape)
    layer = Layer(m, dev, wl, max_tokens=40)
    ids = np.tile(np.array([[5, 2]], np.int32), (40, 1))
    out = layer.forward(wl.x, ids, wl.probs)
    _stage_checks(orc, layer, wl.x, ids, wl.probs, out, 0)
    # K = 1 (top-1): the combine is the identity
    shape1 = W.MoEShape(T=24, H=256, E=8, K=1, I=128)
    wl1 = W.MoEWorkload("top1", 10, shape1)
    layer1 = Layer(m, dev, wl1, max_tokens=24)
    out1 = layer1.forward(wl1.x, wl1.ids, wl1.probs)
    _stage_checks(orc, layer1, wl1.x, wl1.ids, wl1.probs, out1, 0)


@pytest.mark.parametrize("shape", [
    W.MoEShape(T=50, H=128, E=1, K=1, I=128),   # one expert; one 128-column K step in both GEMMs;
                                                # FC2's 128 output columns leave two of four waves idle
    W.MoEShape(T=37, H=384, E=5, K=5, I=384),   # every token to every expert (K = E); 3 K steps;
                                                # FC2 N = 384: a half-filled column tile
    W.MoEShape(T=70, H=640, E=6, K=3, I=256),   # 5 K steps in FC1, 2 in FC2; FC2 N = 640
])
def test_unusual_shapes_all_stages(gpu, orc, shape):
    """Layer shapes away from the workloads: K-step counts of 1, 2, 3, 5; column
    tiles with idle waves; a single expert; K = E."""
    m, dev = gpu
    wl = W.MoEWorkload(f"shape_H{shape.H}_I{shape.I}_E{shape.E}_K{shape.K}", 12, shape)
    layer = Layer(m, dev, wl, max_tokens=shape.T)
    out = layer.forward(wl.x, wl.ids, wl.probs)
    _stage_checks(orc, layer, wl.x, wl.ids, wl.probs, out, 0)
    assert m.device_error(layer.cfg, layer.ws) == 0


def test_zero_tokens_is_noop(gpu):
    import torch
    m, dev = gpu
    wl = W.tiny(seed=0)
    layer = Layer(m, dev, wl, max_tokens=8)
    out = torch.full((1, wl.shape.H), 7, dtype=torch.int16, device=dev)
    st = m.lib().nvfp4moe_moe_expert_forward(ctypes.byref(layer.cfg), None, 0, None, None,
                                             ctypes.byref(layer.qw.W1q), ctypes.byref(layer.qw.W2q), None,
                                             ctypes.c_void_p(layer.ws.data_ptr()), layer.ws.numel(), None)
    torch.cuda.synchronize()
    assert st == 0 and int(out[0, 0]) == 7


def test_device_error_word(gpu):
    """Out-of-range and repeated expert ids set the error word; nothing faults."""
    m, dev = gpu
    wl = W.tiny(seed=0)
    layer = Layer(m, dev, wl, max_tokens=64)
    ids = wl.ids.copy()
    ids[3, 1] = 8
    layer.forward(wl.x, ids, wl.probs)
    assert m.device_error(layer.cfg, layer.ws) & 1
    ids = wl.ids.copy()
    ids[5, 1] = ids[5, 0]
    layer.forward(wl.x, ids, wl.probs)
    assert m.device_error(layer.cfg, layer.ws) == 2
    layer.forward(wl.x, wl.ids, wl.probs)
    assert m.device_error(layer.cfg, layer.ws) == 0


def test_dense_linear(gpu, orc):
    """Dense NVFP4 linear: X [4096, 2048] with 1% outliers x50, W [1536, 2048]."""
    import torch
    m, dev = gpu
    wl = W.dense(seed=1)
    wc, ws_, wg = m.quantize(to_dev(wl.w, dev), layout=m.LAYOUT_GEMM)
    Wq = m.qtensor(wc, ws_, wg, 1, wl.N, wl.K)
    ws = torch.empty((m.linear_workspace_bytes(wl.M, wl.K),), dtype=torch.uint8, device=dev)
    out = to_host(m.linear(to_dev(wl.x, dev), Wq, ws))
    torch.cuda.synchronize()
    ref = orc.linear(orc.quantize(wl.x), orc.quantize(wl.w))
    rel, mx = rel_l2(out, ref)
    print(f"  dense linear rel L2 {rel:.2e} max-abs {mx:.3e}")
    assert rel <= REL_L2_TOL
    # ragged row count
    M = 1000
    out = to_host(m.linear(to_dev(wl.x[:M], dev), Wq, ws))
    torch.cuda.synchronize()
    rel, _ = rel_l2(out, ref[:M])
    assert rel <= REL_L2_TOL


@pytest.fixture(scope="module")
def qwen3_layer(gpu):
    m, dev = gpu
    wl = W.qwen3(seed=2)
    return Layer(m, dev, wl, max_tokens=wl.shape.T)


def test_qwen3_layer_sampled_tokens(gpu, orc, qwen3_layer):
    """Qwen3-30B-A3B-shaped layer, 4096 tokens: sort and A1 in full, outputs on sampled tokens."""
    layer = qwen3_layer
    wl = layer.wl
    T = wl.shape.T
    out = layer.forward(wl.x, wl.ids, wl.probs)
    _, pair2row = _check_route(orc, layer, wl.ids, T)
    _check_a1(orc, layer, wl.x, pair2row, 0)
    sample = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(0).choice(T, 13, replace=False)]))
    ref = _oracle_subset(orc, layer, wl.x[sample], wl.ids[sample], wl.probs[sample])
    rel, mx = rel_l2(out[sample], ref)
    print(f"  qwen3 T=4096 sampled {sample.size} tokens: rel L2 {rel:.2e} max-abs {mx:.3e}")
    assert rel <= REL_L2_TOL
    # the combine is bit-exact on the GPU's own y2 for every token
    s, lay = layer.s, layer.lay
    y2 = layer.ws_array(lay.y2, np.uint16, int(lay.rows_cap) * s.H).reshape(-1, s.H)[pair2row]
    assert np.array_equal(orc.combine(y2.reshape(T, s.K, s.H)), out)


def test_skewed_layer_sampled_tokens(gpu, orc):
    """Zipf(1.1)-skewed routing, 16384 tokens: hottest expert ~15.9k rows, some with <= 8."""
    m, dev = gpu
    wl = W.skewed(seed=3)
    layer = Layer(m, dev, wl, max_tokens=wl.shape.T)
    T = wl.shape.T
    out = layer.forward(wl.x, wl.ids, wl.probs)
    _check_route(orc, layer, wl.ids, T)
    cnt = wl.expert_counts()
    hot, cold = int(np.argmax(cnt)), int(np.argmin(cnt))
    tok_hot = np.where((wl.ids == hot).any(axis=1))[0][[0, -1]]
    tok_cold = np.where((wl.ids == cold).any(axis=1))[0]
    sample = np.unique(np.concatenate([tok_hot, tok_cold, np.random.default_rng(1).choice(T, 8, replace=False)]))
    ref = _oracle_subset(orc, layer, wl.x[sample], wl.ids[sample], wl.probs[sample])
    rel, mx = rel_l2(out[sample], ref)
    print(f"  skewed T=16384 sampled {sample.size} tokens (hot {cnt[hot]}, cold {cnt[cold]}): rel {rel:.2e}")
    assert rel <= REL_L2_TOL


def test_determinism_outputs_and_intermediates(gpu, qwen3_layer):
    layer = qwen3_layer
    wl = layer.wl
    lay, s = layer.lay, layer.s
    o1 = layer.forward(wl.x, wl.ids, wl.probs)
    rows = int(layer.ws_array(lay.expert_off, np.int32, s.E + 1)[-1])
    p2r = layer.ws_array(lay.pair2row, np.int32, wl.shape.T * s.K).copy()
    snap = {k: layer.ws_array(getattr(lay, k), np.uint16, rows * n).reshape(rows, n)[p2r].copy()
            for k, n in (("h", s.I), ("y2", s.H))}
    o2 = layer.forward(wl.x, wl.ids, wl.probs)
    assert np.array_equal(o1, o2)
    for k, n in (("h", s.I), ("y2", s.H)):
        assert np.array_equal(layer.ws_array(getattr(lay, k), np.uint16, rows * n).reshape(rows, n)[p2r], snap[k]), k


def test_batch_invariance_sweep(gpu):
    """Probe tokens alone, in decode batches of every size 1..256 and inside a
    32768-token prefill: each probe's BF16 output is bitwise identical."""
    m, dev = gpu
    pool = W.InvariancePool(seed=4, n_probe=512)
    layer = Layer(m, dev, pool.layer, max_tokens=32768)
    ref = np.stack([layer.forward(pool.x[i:i + 1], pool.ids[i:i + 1], pool.probs[i:i + 1])[0]
                    for i in range(0, 512, 8)])  # every 8th probe alone
    probe_ids = np.arange(0, 512, 8)
    rng = np.random.default_rng(4)
    bad = 0
    for b in range(1, 257):
        probes = rng.choice(probe_ids.size, min(b, 4), replace=False)
        x, ids, probs, pos = pool.batch(b, probe_ids[probes], rng)
        out = layer.forward(x, ids, probs)
        for p, j in zip(pos, probes):
            bad += int(not np.array_equal(out[p], ref[j]))
    x, ids, probs, pos = pool.batch(32768, probe_ids, rng)
    out = layer.forward(x, ids, probs)
    for p, j in zip(pos, range(probe_ids.size)):
        bad += int(not np.array_equal(out[p], ref[j]))
    assert bad == 0, f"{bad} probe outputs differ from their batch-1 bits"


def test_selftest_entry_point(gpu):
    """The exported bitwise self-test on the Qwen3-30B-A3B layer shape."""
    m, dev = gpu
    wl = W.qwen3(seed=4, T=8)
    layer = Layer(m, dev, wl, max_tokens=2048)
    st, rep = m.selftest_batch_invariance(layer.cfg, layer.qw, seed=7, n_probe=32, max_decode_batch=64,
                                          prefill_tokens=2048)
    print("  selftest report", rep)
    assert st == 0 and rep["n_mismatched"] == 0
    assert rep["n_compared"] == sum(min(b, 4) for b in range(1, 65)) + 2 * 32  # prefill: both layouts


def test_weight_reload_in_place(gpu, orc):
    """Re-quantizing new weights into the same buffers gives the same bits as a fresh context."""
    import torch
    m, dev = gpu
    wl_a = W.tiny(seed=0)
    wl_b = W.tiny(seed=11)
    la = Layer(m, dev, wl_a, max_tokens=64)
    out_a = la.forward(wl_a.x, wl_a.ids, wl_a.probs)
    w1b, w2b = wl_b.weights(threads=4)
    la.qw.quantize_from(to_dev(w1b, dev), to_dev(w2b, dev))
    torch.cuda.synchronize()
    out_b_inplace = la.forward(wl_a.x, wl_a.ids, wl_a.probs)
    lb = Layer(m, dev, wl_a, max_tokens=64, weights=(w1b, w2b))
    assert np.array_equal(out_b_inplace, lb.forward(wl_a.x, wl_a.ids, wl_a.probs))
    la.qw.quantize_from(to_dev(la.w1, dev), to_dev(la.w2, dev))
    torch.cuda.synchronize()
    assert np.array_equal(la.forward(wl_a.x, wl_a.ids, wl_a.probs), out_a)
