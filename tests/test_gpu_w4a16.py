"""GPU parity of the W4A16 expert forward (NVFP4 weights, BF16 activations;
the article, section 6: NVFP4 W4A16 routed experts) against the CPU oracle,
through the C ABI.

Bars, as for the W4A4 forward: the expert sort bit-exact; h, y2 and the
outputs within relative L2 <= 1e-2 of the oracle (max-abs reported); the
combine bit-exact on the GPU's own y2; every token's output bitwise the same
alone and inside a full batch."""
import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import rel_l2, to_dev, to_host

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
    def __init__(self, m, dev, wl, max_tokens):
        s = wl.shape
        self.m, self.dev, self.wl, self.s = m, dev, wl, s
        self.w1, self.w2 = wl.weights(threads=16)
        self.cfg = m.make_config(s.H, s.I, s.E, s.K, max_tokens)
        self.qw = m.QuantWeights(self.cfg, dev).quantize_from(to_dev(self.w1, dev), to_dev(self.w2, dev))
        self.ws = m.alloc_workspace(self.cfg, dev)
        self.lay = m.workspace_layout(self.cfg)

    def forward(self, x, ids, probs):
        import torch
        out = self.m.moe_expert_forward_w4a16(self.cfg, to_dev(x, self.dev), to_dev(ids, self.dev),
                                              to_dev(probs, self.dev), self.qw, self.ws)
        torch.cuda.synchronize()
        assert self.m.device_error(self.cfg, self.ws) == 0
        return to_host(out)

    def rows(self, off, n_cols, pair2row):
        rows = int(self.lay.rows_cap)
        a = to_host(self.ws[off:off + rows * n_cols * 2]).view(np.uint16).reshape(rows, n_cols)
        return a[pair2row]

    def pair2row(self, P):
        return to_host(self.ws[self.lay.pair2row:self.lay.pair2row + 4 * P]).view(np.int32)


def _oracle(orc, layer, x, ids, probs, intermediates=False):
    used = np.unique(ids)
    remap = np.full(layer.s.E, -1, np.int32)
    remap[used] = np.arange(used.size)
    wts = orc.DequantWeights(layer.w1[used], layer.w2[used])
    return orc.moe_forward_w4a16(x, remap[ids], probs, wts, intermediates=intermediates)


def _all_stages(orc, layer, x, ids, probs):
    s = layer.s
    T = x.shape[0]
    out = layer.forward(x, ids, probs)
    off, want_p2r, _ = orc.route(ids, s.E, 32)
    p2r = layer.pair2row(T * s.K)
    assert np.array_equal(p2r, want_p2r), "pair -> sorted row"
    ref, mid = _oracle(orc, layer, x, ids, probs, intermediates=True)
    h = layer.rows(layer.lay.h, s.I, p2r)
    y2 = layer.rows(layer.lay.y2, s.H, p2r)
    rel_h, _ = rel_l2(h, mid["h"])
    rel_y2, _ = rel_l2(y2, mid["y2"])
    assert rel_h <= REL_L2_TOL and rel_y2 <= REL_L2_TOL, (rel_h, rel_y2)
    assert np.array_equal(orc.combine(y2.reshape(T, s.K, s.H)), out), "combine of the GPU's y2"
    rel, mx = rel_l2(out, ref)
    print(f"  w4a16 T={T}: h rel {rel_h:.2e}, y2 rel {rel_y2:.2e}, out rel {rel:.2e} max-abs {mx:.3e}")
    assert rel <= REL_L2_TOL
    return out


@pytest.mark.parametrize("shape", [
    W.MoEShape(T=64, H=256, E=8, K=2, I=128),
    W.MoEShape(T=37, H=384, E=5, K=5, I=384),   # K = E; 3 K steps; FC2's last column tile half idle
    W.MoEShape(T=50, H=128, E=1, K=1, I=128),   # one expert, one K step
])
def test_w4a16_all_stages(gpu, orc, shape):
    m, dev = gpu
    wl = W.MoEWorkload(f"w4a16_H{shape.H}", 13, shape)
    layer = Layer(m, dev, wl, shape.T)
    _all_stages(orc, layer, wl.x, wl.ids, wl.probs)
    # ragged token counts reuse the same workspace
    for T in (1, 7):
        _all_stages(orc, layer, wl.x[:T], wl.ids[:T], wl.probs[:T])


def test_w4a16_qwen3_sampled_tokens_and_batch_invariance(gpu, orc):
    m, dev = gpu
    wl = W.qwen3(seed=2)
    layer = Layer(m, dev, wl, wl.shape.T)
    T = wl.shape.T
    out = layer.forward(wl.x, wl.ids, wl.probs)
    sample = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(0).choice(T, 13, replace=False)]))
    ref = _oracle(orc, layer, wl.x[sample], wl.ids[sample], wl.probs[sample])
    rel, mx = rel_l2(out[sample], ref)
    print(f"  w4a16 qwen3 T=4096 sampled {sample.size} tokens: rel L2 {rel:.2e} max-abs {mx:.3e}")
    assert rel <= REL_L2_TOL
    # each sampled token alone, and the sample as one small batch: the same bits
    for t in sample[:6]:
        alone = layer.forward(wl.x[t:t + 1], wl.ids[t:t + 1], wl.probs[t:t + 1])
        assert np.array_equal(alone[0], out[t]), f"token {t} alone"
    small = layer.forward(wl.x[sample], wl.ids[sample], wl.probs[sample])
    assert np.array_equal(small, out[sample])
    # deterministic
    assert np.array_equal(layer.forward(wl.x, wl.ids, wl.probs), out)
