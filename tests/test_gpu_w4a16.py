"""GPU parity of the W4A16 expert forward (NVFP4 weights, BF16 activations;
the article, section 6: NVFP4 W4A16 routed experts) against the CPU oracle,
through the C ABI, element by element (tests/layer_parity.py,
parity_w4a16): the expert sort bit-exact; h within the bound propagated
from FC1's FP32-accumulation bound through the producer; y2 within the FC2
bound of the oracle's FC2 on the GPU's h; the combine bit-exact on the GPU's
own y2; every token's output within the composed bound and relative L2
<= 1e-2; every token's output bitwise the same alone and inside a full batch."""
import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import to_dev, to_host
from tests.layer_parity import parity_w4a16

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


def _all_stages(orc, layer, x, ids, probs, label):
    out = layer.forward(x, ids, probs)
    parity_w4a16(orc, layer.s, layer.lay, layer.ws, x, ids, probs, out, layer.w1, layer.w2, label=label)
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
    _all_stages(orc, layer, wl.x, wl.ids, wl.probs, f"w4a16 H{shape.H} T={shape.T}")
    # ragged token counts reuse the same workspace
    for T in (1, 7):
        _all_stages(orc, layer, wl.x[:T], wl.ids[:T], wl.probs[:T], f"w4a16 H{shape.H} T={T}")


def test_w4a16_qwen3_all_tokens_and_batch_invariance(gpu, orc):
    """Qwen3-30B-A3B-shaped layer, 4096 tokens: every token element-wise against
    the oracle; sampled tokens alone and as a small batch: the same bits."""
    m, dev = gpu
    wl = W.qwen3(seed=2)
    layer = Layer(m, dev, wl, wl.shape.T)
    T = wl.shape.T
    out = _all_stages(orc, layer, wl.x, wl.ids, wl.probs, "w4a16 qwen3 T=4096")
    sample = np.unique(np.concatenate([[0, 1, T - 1], np.random.default_rng(0).choice(T, 13, replace=False)]))
    # each sampled token alone, and the sample as one small batch: the same bits
    for t in sample[:6]:
        alone = layer.forward(wl.x[t:t + 1], wl.ids[t:t + 1], wl.probs[t:t + 1])
        assert np.array_equal(alone[0], out[t]), f"token {t} alone"
    small = layer.forward(wl.x[sample], wl.ids[sample], wl.probs[sample])
    assert np.array_equal(small, out[sample])
    # deterministic
    assert np.array_equal(layer.forward(wl.x, wl.ids, wl.probs), out)
