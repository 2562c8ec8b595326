"""The masked fixed-capacity row layout against the contiguous one (article,
section 4.4, "two layouts, same row results": the decode side's per-expert
chunks of fixed capacity and the training side's packed rows must give every
(token, slot) the same bits).

Per workload and capacity, through the C ABI:
  - device offsets off[e] = e * capacity; counts as in the contiguous layout;
  - pair -> row: e * capacity + the pair's rank within its expert (the rank
    read off the contiguous layout); row -> pair inside each chunk, padding
    rows -1;
  - every expert's rows of A1 (quantized X), h, A2 (quantized h) and y2 hold
    the same bytes in both layouts (with the padding rows of A1 and A2); the
    outputs are equal;
  - an expert with more pairs than the capacity: error bit 4, the pairs past
    the capacity get no row, and every token none of whose pairs was dropped
    keeps its contiguous-layout output bits;
  - against the oracle: the masked sort metadata (offsets, pair -> row,
    row -> pair inside each expert's used rows, dropped pairs) bit-exact with
    the oracle's masked layout, and every stage of the masked forward
    element-wise against the oracle (tests/layer_parity.py)."""
import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import to_dev, to_host
from tests.layer_parity import check_route, parity

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_moe_expert_sort_amd as m
    m.lib()
    return m, torch.device("cuda:0")


def _ws(ws, off, dtype, count):
    return to_host(ws[off:off + count * np.dtype(dtype).itemsize]).view(dtype)


class Run:
    """One forward: its workspace (on the device) and the routing arrays on the host."""

    def __init__(self, m, cfg, lay, ws, out, s):
        self.lay, self.ws, self.s = lay, ws, s
        self.out = to_host(out)
        self.off = _ws(ws, lay.expert_off, np.int32, s.E + 1).astype(np.int64)
        self.cnt = _ws(ws, lay.expert_count, np.int32, s.E).astype(np.int64)
        self.p2r = _ws(ws, lay.pair2row, np.int32, s.T * s.K).astype(np.int64)
        self.r2p = _ws(ws, lay.row2pair, np.int32, int(lay.rows_cap))
        self.err = m.device_error(cfg, ws)

    def rows(self, name, r0, n):
        """Bytes of sorted rows [r0, r0 + n) of one buffer (r0, n multiples of 32 for
        the GEMM-layout planes, whose 32-row tiles are contiguous)."""
        s, lay = self.s, self.lay
        per_row = {"a1_codes": s.H // 2, "a1_scales": s.H // 16, "a1_g": 4, "h": 2 * s.I,
                   "a2_codes": s.I // 2, "a2_scales": s.I // 16, "a2_g": 4, "y2": 2 * s.H}[name]
        base = getattr(lay, name)
        return self.ws[base + r0 * per_row:base + (r0 + n) * per_row]


# planes whose padding rows are written (zeros) and compared with the expert's rows
_PADDED = ("a1_codes", "a1_scales", "a1_g", "a2_codes", "a2_scales", "a2_g")
# planes whose padding rows are never written: only the expert's rows are compared
_VALID = ("h", "y2")


def _both(m, dev, wl, capacity, mode=0):
    import torch
    s = wl.shape
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, s.T, scale_round=mode)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    x, ids, probs = to_dev(wl.x, dev), to_dev(wl.ids, dev), to_dev(wl.probs, dev)
    ws_c = m.alloc_workspace(cfg, dev)
    out_c = m.moe_expert_forward(cfg, x, ids, probs, qw, ws_c)
    ws_m = m.alloc_workspace_masked(cfg, capacity, dev)
    out_m = m.moe_expert_forward_masked(cfg, capacity, x, ids, probs, qw, ws_m)
    torch.cuda.synchronize()
    cont = Run(m, cfg, m.workspace_layout(cfg), ws_c, out_c, s)
    mask = Run(m, cfg, m.workspace_layout_masked(cfg, capacity), ws_m, out_m, s)
    mask.weights = (w1, w2)
    return cont, mask


def _check_experts(cont, mask, capacity):
    """Each expert's rows (the first `capacity` of them when it overflows) hold
    the same bytes in both layouts: an expert's rows start on a 32-row tile in
    both, so its GEMM-layout tiles are byte ranges of the same length."""
    import torch
    for e in range(cont.s.E):
        n = int(min(cont.cnt[e], capacity))
        if n == 0:
            continue
        pad = (n + 31) // 32 * 32
        rc, rm = int(cont.off[e]), e * capacity
        for name in _PADDED:
            assert torch.equal(mask.rows(name, rm, pad), cont.rows(name, rc, pad)), f"{name} of expert {e}"
        for name in _VALID:
            assert torch.equal(mask.rows(name, rm, n), cont.rows(name, rc, n)), f"{name} of expert {e}"


def _check_placement(cont, mask, pairs, capacity, ids):
    e = ids.reshape(-1)[pairs]
    rc, rm = cont.p2r[pairs], mask.p2r[pairs]
    assert np.array_equal(rm, e * capacity + (rc - cont.off[e])), "masked row = e * capacity + rank"
    assert np.array_equal(mask.r2p[rm], pairs), "row -> pair"


@pytest.mark.parametrize("case", ["tiny-RU", "tiny-RNE", "qwen3", "skewed"])
def test_masked_rows_equal_contiguous_rows(gpu, orc, case):
    m, dev = gpu
    wl, capacity, mode = {"tiny-RU": (W.tiny(seed=0), 32, 0), "tiny-RNE": (W.tiny(seed=0), 64, 1),
                          "qwen3": (W.qwen3(seed=2, T=4096), 320, 0),
                          "skewed": (W.skewed(seed=3, T=2048), 2016, 0)}[case]
    s = wl.shape
    cont, mask = _both(m, dev, wl, capacity, mode)
    assert cont.err == 0 and mask.err == 0
    assert np.array_equal(mask.off, np.arange(s.E + 1) * capacity), "device offsets e * capacity"
    assert np.array_equal(mask.cnt, cont.cnt), "expert counts"
    _check_placement(cont, mask, np.arange(s.T * s.K), capacity, wl.ids)
    _check_experts(cont, mask, capacity)
    # each chunk: the expert's rows, then padding rows (-1) up to a multiple of 32
    for e in range(s.E):
        n = int(mask.cnt[e])
        pad = (n + 31) // 32 * 32
        assert np.all(mask.r2p[e * capacity + n:e * capacity + pad] == -1), f"padding rows of expert {e}"
    assert np.array_equal(mask.out, cont.out), "outputs differ between the layouts"
    print(f"  {case}: capacity {capacity}, {s.T * s.K} pairs, every row and output bit-equal")
    # the masked forward against the oracle: metadata bit-exact, every stage element-wise
    lay_m = m.workspace_layout_masked(m.make_config(s.H, s.I, s.E, s.K, s.T, scale_round=mode), capacity)
    parity(orc, s, lay_m, mask.ws, wl.x, wl.ids, wl.probs, mask.out, *mask.weights, mode=mode, capacity=capacity,
           label=f"masked {case}")


def test_masked_capacity_overflow(gpu, orc):
    m, dev = gpu
    wl = W.qwen3(seed=2, T=4096)  # 213..298 pairs per expert
    capacity = 256
    s = wl.shape
    cont, mask = _both(m, dev, wl, capacity)
    assert cont.err == 0 and mask.err == 4, f"error word {mask.err}"
    # metadata against the oracle's masked layout, dropped pairs included
    check_route(orc, s.E, s.K, s.T, m.workspace_layout_masked(m.make_config(s.H, s.I, s.E, s.K, s.T), capacity),
                mask.ws, wl.ids, capacity)
    e = wl.ids.reshape(-1)
    rank = cont.p2r - cont.off[e]
    dropped = rank >= capacity
    assert dropped.any() and not dropped.all()
    assert np.all(mask.p2r[dropped] == -1), "pairs past the capacity get no row"
    _check_placement(cont, mask, np.nonzero(~dropped)[0], capacity, wl.ids)
    _check_experts(cont, mask, capacity)
    tok_ok = ~dropped.reshape(s.T, s.K).any(axis=1)
    assert tok_ok.any()
    assert np.array_equal(mask.out[tok_ok], cont.out[tok_ok]), "tokens with no dropped pair keep their bits"
    # full experts hold exactly `capacity` rows, no padding
    assert np.all(mask.r2p[(np.arange(s.E) * capacity)[cont.cnt > capacity][:, None] + np.arange(capacity)] >= 0)
    print(f"  capacity {capacity}: {int(dropped.sum())} pairs dropped, {int(tok_ok.sum())} of {s.T} tokens unchanged")


def test_masked_capacity_overflow_small_batch(gpu, orc):
    """The same through the single-launch sort (800 pairs): the first 40 of 100
    tokens all route to experts 0..7, which then hold 40 pairs each against a
    capacity of 32."""
    import types
    m, dev = gpu
    base = W.qwen3(seed=2, T=4096)
    T, capacity, s_E = 100, 32, base.shape.E
    ids = base.ids[:T].copy()
    ids[:40] = np.arange(8, dtype=np.int32)[None, :]
    for t in range(40, T):  # the other tokens keep away from experts 0..7
        free = iter(e for e in range(8, s_E) if e not in ids[t])
        ids[t] = [e if e >= 8 else next(free) for e in ids[t]]
    s = W.MoEShape(T=T, H=base.shape.H, E=base.shape.E, K=base.shape.K, I=base.shape.I)
    wl = types.SimpleNamespace(shape=s, x=base.x[:T], ids=ids, probs=base.probs[:T], weights=base.weights)
    cont, mask = _both(m, dev, wl, capacity)
    assert cont.err == 0 and mask.err == 4, f"error word {mask.err}"
    check_route(orc, s.E, s.K, s.T, m.workspace_layout_masked(m.make_config(s.H, s.I, s.E, s.K, s.T), capacity),
                mask.ws, ids, capacity)
    e = ids.reshape(-1)
    rank = cont.p2r - cont.off[e]
    dropped = rank >= capacity
    assert int(dropped.sum()) == 8 * 8
    assert np.all(mask.p2r[dropped] == -1), "pairs past the capacity get no row"
    _check_placement(cont, mask, np.nonzero(~dropped)[0], capacity, ids)
    _check_experts(cont, mask, capacity)
    tok_ok = ~dropped.reshape(s.T, s.K).any(axis=1)
    assert tok_ok.sum() == T - 8
    assert np.array_equal(mask.out[tok_ok], cont.out[tok_ok]), "tokens with no dropped pair keep their bits"
