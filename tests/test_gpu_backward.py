"""GPU parity of the BF16 straight-through backward (miniTE summary page, "how
it differs": quantization taken as the identity, BF16 GEMMs on the stored
original BF16 activations and weights) against the oracle, through the C ABI.

Each step is checked on the GPU's own input to it (tests/parity.py bounds):
  dh            oracle GEMM of dout and W2 -> FP32-accumulation bound, K = H
  dgate | dup   oracle SwiGLU backward of the GPU's dh -> one BF16 ulp
  dprobs        same step -> FP32 sum bound over I terms plus the hardware
                exp/reciprocal's relative error
  dx per pair   oracle GEMM of the GPU's dgate|dup and W1 -> bound, K = 2I
  dx            the combine of the GPU's per-pair gradients -> bit-exact
  dW1, dW2      oracle weight gradients of the GPU's dgate|dup and h -> FP32
                accumulation bound over the expert's rows
and end to end against the oracle's whole backward in relative L2; dx is
bitwise batch-invariant and every output deterministic."""
import numpy as np
import pytest

import moe_workloads as W
from tests import parity as PB
from tests.helpers import rel_l2, to_dev, to_host
from tests.layer_parity import ws_array

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


@pytest.fixture(scope="module")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_moe_expert_sort_amd as m
    m.lib()
    return m, torch.device("cuda:0")


def _f32_check(what, got, ref, bound):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    bad = np.argwhere(err > bound)
    assert bad.size == 0, f"{what}: {bad.shape[0]} out of bound, first {tuple(bad[0])}: {got[tuple(bad[0])]} vs {ref[tuple(bad[0])]}"
    return float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0


def _run(m, dev, wl, T=None, seed=31):
    import torch
    s = wl.shape
    T = s.T if T is None else T
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, T)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    ws = m.alloc_workspace(cfg, dev)
    x, ids, probs = wl.x[:T], wl.ids[:T], wl.probs[:T]
    xd = to_dev(x, dev)
    out, y1 = m.moe_expert_forward_unfused(cfg, xd, to_dev(ids, dev), to_dev(probs, dev), qw, ws)
    rng = np.random.default_rng(seed)
    dout = W.f32_to_bf16_bits((rng.standard_normal((T, s.H)) * 0.1).astype(np.float32))
    dx, dprobs, dw1, dw2, bws = m.moe_expert_backward(cfg, xd, to_dev(w1, dev), to_dev(w2, dev), y1, ws,
                                                      to_dev(dout, dev))
    torch.cuda.synchronize()
    return dict(cfg=cfg, ws=ws, y1=y1, bws=bws, w1=w1, w2=w2, x=x, ids=ids, probs=probs, dout=dout,
                dx=to_host(dx), dprobs=to_host(dprobs), dw1=to_host(dw1), dw2=to_host(dw2))


def _parity(m, orc, wl, label, T=None):
    import torch  # noqa: F401
    dev = __import__("torch").device("cuda:0")
    R = _run(m, dev, wl, T)
    s = wl.shape
    T, H, I, K, E = R["x"].shape[0], s.H, s.I, s.K, s.E
    lay = m.workspace_layout(R["cfg"])
    rows = int(lay.rows_cap)
    p2r = ws_array(R["ws"], lay.pair2row, np.int32, T * K)
    e_pair = R["ids"].reshape(-1)
    y1 = to_host(R["y1"])[p2r]
    h = ws_array(R["ws"], lay.h, np.uint16, rows * I).reshape(rows, I)[p2r]
    nb = m.lib().nvfp4moe_backward_workspace_bytes(__import__("ctypes").byref(R["cfg"]))
    bws = to_host(R["bws"])
    off_dy1 = -(-rows * I * 2 // 256) * 256
    off_dxp = off_dy1 + -(-rows * 2 * I * 2 // 256) * 256
    dh = bws[:rows * I * 2].view(np.uint16).reshape(rows, I)[p2r]
    dy1 = bws[off_dy1:off_dy1 + rows * 2 * I * 2].view(np.uint16).reshape(rows, 2 * I)[p2r]
    dxp = bws[off_dxp:off_dxp + rows * H * 2].view(np.uint16).reshape(rows, H)[p2r]
    assert nb >= off_dxp + rows * H * 2
    w1v = W.bf16_bits_to_f32(R["w1"]).astype(np.float64)
    w2v = W.bf16_bits_to_f32(R["w2"]).astype(np.float64)
    reports = []
    # dh = bf16(dout[t] . W2[e]): column norms of W2[e] over m
    dout = R["dout"]
    dout_pairs = np.repeat(dout, K, axis=0)
    ref_dh = np.empty_like(dh)
    for e in np.unique(e_pair):
        sel = np.nonzero(e_pair == e)[0]
        ref_dh[sel] = orc.gemm_epilogue(PB.vals(dout_pairs[sel]), np.ones(sel.size, np.float32), w2v[e].T.copy(),
                                        np.ones(I, np.float32))
    c = PB.Check(f"{label} dh")
    PB.check_grouped_gemm(c, dh, ref_dh, PB.row_norms(PB.vals(dout_pairs)), np.sqrt((w2v ** 2).sum(axis=1)), e_pair, H)
    reports.append(c.report())
    # SwiGLU backward of the GPU's dh
    ref_dy1, ref_dp = orc.swiglu_backward(dh, y1, R["probs"].reshape(-1))
    c = PB.Check(f"{label} dgate|dup")
    g = PB.vals(y1[:, :I])
    assert g.min() > -64.0
    c.add(dy1, ref_dy1, PB.ulp_bf16(np.maximum(np.abs(PB.vals(dy1)), np.abs(PB.vals(ref_dy1)))))
    reports.append(c.report() + f"; {int((dy1 != ref_dy1).sum())} of {dy1.size} differ")
    terms = np.abs(PB.vals(dh) * (g / (1 + np.exp(-g))) * PB.vals(y1[:, I:])).sum(axis=1)
    w = _f32_check(f"{label} dprobs", R["dprobs"].reshape(-1), ref_dp, (2 * I * U + 1e-6) * terms + 1e-30)
    reports.append(f"{label} dprobs: within bound (worst {w:.3f} of it)")
    # the FC1 input gradient per pair, on the GPU's dgate|dup
    ref_dxp = np.empty_like(dxp)
    for e in np.unique(e_pair):
        sel = np.nonzero(e_pair == e)[0]
        ref_dxp[sel] = orc.gemm_epilogue(PB.vals(dy1[sel]), np.ones(sel.size, np.float32), w1v[e].T.copy(),
                                         np.ones(H, np.float32))
    c = PB.Check(f"{label} dx per pair")
    PB.check_grouped_gemm(c, dxp, ref_dxp, PB.row_norms(PB.vals(dy1)), np.sqrt((w1v ** 2).sum(axis=1)), e_pair, 2 * I)
    reports.append(c.report())
    assert np.array_equal(orc.combine(dxp.reshape(T, K, H)), R["dx"]), "dx = combine of the per-pair gradients"
    # weight gradients on the GPU's dgate|dup and h
    ref_dw1, ref_dw2 = orc.moe_weight_grads(R["x"], dout, R["ids"], dy1, h, E)
    xv, dv, hv, dyv = PB.vals(R["x"]), PB.vals(dout), PB.vals(h), PB.vals(dy1)
    worst = 0.0
    for e in range(E):
        sel = np.nonzero(e_pair == e)[0]
        n = max(sel.size, 1)
        tok = sel // K
        b1 = 2 * n * U * np.sqrt((dyv[sel] ** 2).sum(axis=0))[:, None] * np.sqrt((xv[tok] ** 2).sum(axis=0))[None, :]
        b2 = 2 * n * U * np.sqrt((dv[tok] ** 2).sum(axis=0))[:, None] * np.sqrt((hv[sel] ** 2).sum(axis=0))[None, :]
        worst = max(worst, _f32_check(f"{label} dW1[{e}]", R["dw1"][e], ref_dw1[e], b1 + U * np.abs(ref_dw1[e]) + 1e-30),
                    _f32_check(f"{label} dW2[{e}]", R["dw2"][e], ref_dw2[e], b2 + U * np.abs(ref_dw2[e]) + 1e-30))
    reports.append(f"{label} dW1, dW2: within the FP32 bound (worst {worst:.3f} of it)")
    # end to end against the oracle's whole backward
    odx, odp, odw1, odw2 = orc.moe_backward(R["x"], R["ids"], R["probs"], R["w1"], R["w2"], y1, h, dout)
    rel = {"dx": rel_l2(R["dx"], odx)[0]}
    for name, got, ref in (("dprobs", R["dprobs"], odp), ("dW1", R["dw1"], odw1), ("dW2", R["dw2"], odw2)):
        g64, r64 = got.astype(np.float64), ref.astype(np.float64)
        rel[name] = float(np.linalg.norm(g64 - r64) / max(np.linalg.norm(r64), 1e-300))
    reports.append(f"{label} end to end vs the oracle's backward, relative L2: " +
                   ", ".join(f"{k} {v:.2e}" for k, v in rel.items()))
    assert all(v <= 1e-2 for v in rel.values()), reports[-1]
    print("\n  " + "\n  ".join(reports))
    return R


SMALL_CASES = {
    "H384_I384_E5_K5": W.MoEShape(T=37, H=384, E=5, K=5, I=384),  # every token to every expert
    "H256_I640_E3_K2": W.MoEShape(T=450, H=256, E=3, K=2, I=640),  # a partial 256-column tile (640)
    "H256_I256_E4_K1": W.MoEShape(T=300, H=256, E=4, K=1, I=256),  # top-1 routing
    "H128_I128_E1_K1": W.MoEShape(T=200, H=128, E=1, K=1, I=128),  # one expert takes every token
}


@pytest.mark.parametrize("case", ["tiny", *SMALL_CASES])
def test_backward_small(gpu, orc, case):
    m, dev = gpu
    wl = W.tiny(seed=0) if case == "tiny" else W.MoEWorkload(case, 12, SMALL_CASES[case])
    _parity(m, orc, wl, case)


def test_backward_ragged_and_invariant(gpu, orc):
    """T = 1, 17 and 64 of the tiny layer; each token's dx is bitwise the same
    alone as in the batch, and two runs give the same bits."""
    m, dev = gpu
    wl = W.tiny(seed=5)
    full = _run(m, dev, wl)
    for T in (1, 17):
        part = _parity(m, orc, wl, f"tiny T={T}", T=T)
        assert np.array_equal(part["dx"], full["dx"][:T]), f"dx of the first {T} tokens"
    again = _run(m, dev, wl)
    for k in ("dx", "dprobs", "dw1", "dw2"):
        assert np.array_equal(again[k].view(np.uint8), full[k].view(np.uint8)), k


def test_backward_qwen3_layer(gpu, orc):
    """Qwen3-30B-A3B-shaped layer, 4096 tokens: every step of every pair."""
    m, dev = gpu
    _parity(m, orc, W.qwen3(seed=2), "qwen3 T=4096")


def test_backward_skewed(gpu, orc):
    """Zipf(1.1) expert popularity at the Qwen3 shape, T = 2048: the hottest
    expert holds 1978 rows (weight-gradient K loops of 31 chunks, many row
    tiles of one expert in dh and the FC1 input gradient) and 9 experts none
    (their weight gradients are zeros)."""
    m, dev = gpu
    wl = W.skewed(seed=3, T=2048)
    counts = wl.expert_counts()
    assert counts.max() == 1978 and (counts == 0).sum() == 9
    R = _parity(m, orc, wl, "skewed T=2048")
    empty = np.nonzero(counts == 0)[0]
    assert not R["dw1"][empty].any() and not R["dw2"][empty].any()
