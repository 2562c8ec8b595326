"""GPU parity of the NVFP4 MoE expert forward and the dense NVFP4 linear,
through the C ABI, against the CPU oracle, element by element.

Every stage is compared on the GPU's own input to it (tests/layer_parity.py):
integer and byte work (the expert sort, device offsets, quantized buffers,
the FC2 maxima, the combine of the GPU's expert outputs) bit-exact; FC1's y1
(from the unfused forward, whose h is bitwise the fused forward's) and FC2's
y2 within the FP32-accumulation bound of the FP64 oracle (tests/parity.py);
h within one BF16 ulp of the FP64 producer on the same y1; the output of
every token within the bound composed from those, and relative L2 <= 1e-2.
All tokens of every workload are compared, the Qwen3-30B-A3B-shaped layer
(4096 tokens) and the skewed one (16384) included.
Sources: miniTE summary page, "how it differs" and "how to use it"; article
sections 4.4 and 4.5."""
import ctypes

import numpy as np
import pytest

import moe_workloads as W
from tests import parity as PB
from tests.helpers import rel_l2, to_dev, to_host
from tests.layer_parity import parity

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
        self.m, self.dev, self.wl, self.s, self.mode = m, dev, wl, s, mode
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

    def forward_unfused(self, x, ids, probs):
        import torch
        out, y1 = self.m.moe_expert_forward_unfused(self.cfg, to_dev(x, self.dev), to_dev(ids, self.dev),
                                                    to_dev(probs, self.dev), self.qw, self.ws)
        torch.cuda.synchronize()
        return to_host(out), to_host(y1)

    def ws_array(self, off, dtype, count):
        a = to_host(self.ws[off:off + count * np.dtype(dtype).itemsize])
        return a.view(dtype)

    def check(self, orc, x, ids, probs, label, unfused=True):
        """Unfused forward (y1), then the fused forward; parity of every stage of the
        fused forward's workspace, with the unfused y1 for FC1.  The fused and
        unfused outputs and intermediates are compared bit for bit elsewhere
        (tests/test_gpu_unfused.py); here the unfused output must equal the fused."""
        y1 = None
        if unfused:
            out_u, y1 = self.forward_unfused(x, ids, probs)
        out = self.forward(x, ids, probs)
        if unfused:
            assert np.array_equal(out_u, out), "unfused and fused outputs differ"
        parity(orc, self.s, self.lay, self.ws, x, ids, probs, out, self.w1, self.w2, self.mode, y1_rows=y1,
               label=label)
        assert self.m.device_error(self.cfg, self.ws) == 0
        return out


@pytest.mark.parametrize("mode", [0, 1])
def test_tiny_layer_all_stages(gpu, orc, mode):
    m, dev = gpu
    wl = W.tiny(seed=0)
    layer = Layer(m, dev, wl, max_tokens=wl.shape.T, mode=mode)
    layer.check(orc, wl.x, wl.ids, wl.probs, f"tiny mode {mode}")


def test_tiny_layer_ragged_batches(gpu, orc):
    """Token counts that leave partial tiles everywhere: 1, 3, 17, 33, 64."""
    m, dev = gpu
    wl = W.tiny(seed=5)
    layer = Layer(m, dev, wl, max_tokens=64)
    for T in (1, 3, 17, 33, 64):
        layer.check(orc, wl.x[:T], wl.ids[:T], wl.probs[:T], f"tiny T={T}")


def test_routing_edge_cases(gpu, orc):
    """Every token to the same experts; experts with no tokens; K = 1."""
    m, dev = gpu
    shape = W.MoEShape(T=40, H=256, E=8, K=2, I=128)
    wl = W.MoEWorkload("edge", 9, shape)
    layer = Layer(m, dev, wl, max_tokens=40)
    ids = np.tile(np.array([[5, 2]], np.int32), (40, 1))
    layer.check(orc, wl.x, ids, wl.probs, "all tokens to experts 5, 2")
    # K = 1 (top-1): the combine is the identity
    shape1 = W.MoEShape(T=24, H=256, E=8, K=1, I=128)
    wl1 = W.MoEWorkload("top1", 10, shape1)
    layer1 = Layer(m, dev, wl1, max_tokens=24)
    layer1.check(orc, wl1.x, wl1.ids, wl1.probs, "top-1")


@pytest.mark.parametrize("shape", [
    W.MoEShape(T=50, H=128, E=1, K=1, I=128),   # one expert; one 128-column K step in both GEMMs;
                                                # FC2's 128 output columns leave two of four waves idle
    W.MoEShape(T=37, H=384, E=5, K=5, I=384),   # every token to every expert (K = E); 3 K steps;
                                                # FC2 N = 384: a half-filled column tile
    W.MoEShape(T=70, H=640, E=6, K=3, I=256),   # 5 K steps in FC1, 2 in FC2; FC2 N = 640
    W.MoEShape(T=450, H=256, E=3, K=2, I=640),  # about 300 rows per expert: 3 row tiles each, the
                                                # last partial; I = 640: 5 FC1 column tiles, 5 FC2 K steps
    W.MoEShape(T=40, H=4224, E=4, K=2, I=128),  # the sort's quantizer holds 3 groups per lane (idle lanes in
                                                # the last); 33 FC1 K steps; FC2 N = 4224: a half column tile
    W.MoEShape(T=24, H=8320, E=3, K=2, I=128),  # rows wider than 8192 columns: the quantizer's wave loop
    W.MoEShape(T=150, H=4224, E=4, K=2, I=128),  # the same two widths past 128 tokens, where the block-wise
    W.MoEShape(T=150, H=8320, E=3, K=2, I=128),  # sort (not the single-launch one) quantizes X
])
def test_unusual_shapes_all_stages(gpu, orc, shape):
    """Layer shapes away from the workloads: K-step counts of 1, 2, 3, 5, 33, 65;
    column tiles with idle waves; a single expert; K = E; several row tiles per
    expert; token rows too wide for the quantizer's registers."""
    m, dev = gpu
    wl = W.MoEWorkload(f"shape_H{shape.H}_I{shape.I}_E{shape.E}_K{shape.K}", 12, shape)
    layer = Layer(m, dev, wl, max_tokens=shape.T)
    layer.check(orc, wl.x, wl.ids, wl.probs, f"H{shape.H} I{shape.I} E{shape.E} K{shape.K}")


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
    """Dense NVFP4 linear: X [4096, 2048] with 1% outliers x50, W [1536, 2048];
    every element within the FP32-accumulation bound of the oracle, and a
    ragged row count."""
    import torch
    m, dev = gpu
    wl = W.dense(seed=1)
    wc, ws_, wg = m.quantize(to_dev(wl.w, dev), layout=m.LAYOUT_GEMM)
    Wq = m.qtensor(wc, ws_, wg, 1, wl.N, wl.K)
    ws = torch.empty((m.linear_workspace_bytes(wl.M, wl.K),), dtype=torch.uint8, device=dev)
    out = to_host(m.linear(to_dev(wl.x, dev), Wq, ws))
    torch.cuda.synchronize()
    xq, wq = orc.quantize(wl.x), orc.quantize(wl.w)
    ref = orc.linear(xq, wq)
    xn = PB.row_norms(orc.dequantize(xq[0], xq[1])) * xq[2]
    wn = PB.row_norms(orc.dequantize(wq[0], wq[1])) * wq[2]
    chk = PB.Check("dense linear")
    for i0 in range(0, wl.M, 1024):
        sl = slice(i0, i0 + 1024)
        chk.add(out[sl], ref[sl], PB.gemm_bound(ref[sl], out[sl], xn[sl], wn, wl.K), index_offset=i0)
    rel, mx = rel_l2(out, ref)
    print(f"  {chk.report()}; rel L2 {rel:.2e} max-abs {mx:.3e}")
    assert rel <= REL_L2_TOL
    # ragged row count: the same rows, bit for bit (rows are independent)
    M = 1000
    out_r = to_host(m.linear(to_dev(wl.x[:M], dev), Wq, ws))
    torch.cuda.synchronize()
    assert np.array_equal(out_r, out[:M])
    # three times the rows: enough row tiles for the 256-column tiles (4096 rows
    # take the 128-column ones); the width changes no bit
    xb = np.concatenate([wl.x] * 3)
    wsb = torch.empty((m.linear_workspace_bytes(xb.shape[0], wl.K),), dtype=torch.uint8, device=dev)
    out_b = to_host(m.linear(to_dev(xb, dev), Wq, wsb))
    torch.cuda.synchronize()
    for i in range(3):
        assert np.array_equal(out_b[i * wl.M:(i + 1) * wl.M], out)


@pytest.fixture(scope="module")
def qwen3_layer(gpu):
    m, dev = gpu
    wl = W.qwen3(seed=2)
    return Layer(m, dev, wl, max_tokens=wl.shape.T)


def test_qwen3_layer_all_tokens(gpu, orc, qwen3_layer):
    """Qwen3-30B-A3B-shaped layer, 4096 tokens: every stage of every token and
    pair element-wise against the oracle (32768 pairs, 128 experts)."""
    wl = qwen3_layer.wl
    qwen3_layer.check(orc, wl.x, wl.ids, wl.probs, "qwen3 T=4096")


def test_qwen3_sort_path_boundary(gpu, orc, qwen3_layer):
    """The sort runs in one workgroup up to 1024 pairs and block-wise beyond:
    the first 1, 8, 128 (1024 pairs) and 129 tokens of the layer, every stage
    against the oracle, and each token's output bitwise the same on both sides
    of the boundary."""
    wl = qwen3_layer.wl
    outs = {}
    for T in (1, 8, 128, 129):
        outs[T] = qwen3_layer.check(orc, wl.x[:T], wl.ids[:T], wl.probs[:T], f"qwen3 T={T}")
    for T in (1, 8, 128):
        assert np.array_equal(outs[T], outs[129][:T]), f"first {T} tokens"


def test_device_error_word_blockwise_sort(gpu, qwen3_layer):
    """The error word from the block-wise sort (more than 1024 pairs): an
    out-of-range id sets bit 1, a repeated id bit 2, and a clean batch none."""
    m = qwen3_layer.m
    wl = qwen3_layer.wl
    T = 200
    ids = wl.ids[:T].copy()
    ids[150, 3] = wl.shape.E
    qwen3_layer.forward(wl.x[:T], ids, wl.probs[:T])
    assert m.device_error(qwen3_layer.cfg, qwen3_layer.ws) & 1
    ids = wl.ids[:T].copy()
    ids[170, 5] = ids[170, 2]
    qwen3_layer.forward(wl.x[:T], ids, wl.probs[:T])
    assert m.device_error(qwen3_layer.cfg, qwen3_layer.ws) == 2
    qwen3_layer.forward(wl.x[:T], wl.ids[:T], wl.probs[:T])
    assert m.device_error(qwen3_layer.cfg, qwen3_layer.ws) == 0


def test_skewed_layer_all_tokens(gpu, orc):
    """Zipf(1.1)-skewed routing, 16384 tokens (hottest expert ~15.9k rows, some
    with <= 8): every stage of every token element-wise against the oracle."""
    m, dev = gpu
    wl = W.skewed(seed=3)
    layer = Layer(m, dev, wl, max_tokens=wl.shape.T)
    cnt = wl.expert_counts()
    print(f"  expert rows: min {cnt.min()}, max {cnt.max()}")
    layer.check(orc, wl.x, wl.ids, wl.probs, "skewed T=16384")


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
    """Each of the 512 probe tokens alone (512 forwards of T = 1) and all 512
    inside one 32768-token prefill; decode batches of every size b = 1..256,
    each holding min(b, 4) probes drawn at random from the 512 at random
    positions among filler tokens (1018 probe placements).  Every probe's BF16
    output is bitwise its batch-1 output."""
    m, dev = gpu
    pool = W.InvariancePool(seed=4, n_probe=512)
    layer = Layer(m, dev, pool.layer, max_tokens=32768)
    ref = np.stack([layer.forward(pool.x[i:i + 1], pool.ids[i:i + 1], pool.probs[i:i + 1])[0]
                    for i in range(512)])
    probe_ids = np.arange(512)
    rng = np.random.default_rng(4)
    bad = compared = 0
    for b in range(1, 257):
        probes = rng.choice(probe_ids.size, min(b, 4), replace=False)
        x, ids, probs, pos = pool.batch(b, probe_ids[probes], rng)
        out = layer.forward(x, ids, probs)
        for p, j in zip(pos, probes):
            bad += int(not np.array_equal(out[p], ref[j]))
            compared += 1
    x, ids, probs, pos = pool.batch(32768, probe_ids, rng)
    out = layer.forward(x, ids, probs)
    for p, j in zip(pos, range(probe_ids.size)):
        bad += int(not np.array_equal(out[p], ref[j]))
        compared += 1
    print(f"  {compared} probe outputs compared with their batch-1 bits, {bad} differ")
    assert compared == sum(min(b, 4) for b in range(1, 257)) + 512
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
