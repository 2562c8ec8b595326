"""GPU router (scores + deterministic top-k) against the CPU oracle, through the
C ABI (article, section 4.4, "R3 unnecessary": one FP32-output scoring kernel
for every batch size; section 2: same tie-breaking and output order).

Bars:
  - scores within the FP32 accumulation bound of the exact value:
    |l - l_exact| <= H * 2^-24 * sum_h |x_h w_h| (the worst-case bound for a
    length-H FP32 sum of exact products);
  - ids bit-exact against the oracle's top-k of the GPU's own scores (the
    discrete choice taken on the same FP32 values on both sides);
  - probabilities within (n + 8) * 2^-24 relative (n = the terms of the FP32
    softmax denominator: K or E; FP32 exp, sum and division);
  - bitwise batch invariance of scores, ids and probabilities;
  - exact ties go to the lower expert id."""
import numpy as np
import pytest

import moe_workloads as W
import oracle
from tests.helpers import to_dev, to_host

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


def _router_weights(E, H, seed):
    rng = np.random.default_rng(seed)
    return W.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.02).astype(np.float32))


def _check(m, dev, x, w, k, renorm):
    logits, ids, probs = m.router_topk(to_dev(x, dev), to_dev(w, dev), k, renormalize=renorm)
    logits, ids, probs = to_host(logits), to_host(ids), to_host(probs)
    exact = oracle.router_logits(x, w)
    bound = x.shape[1] * U * (np.abs(W.bf16_bits_to_f32(x).astype(np.float64)) @
                              np.abs(W.bf16_bits_to_f32(w).astype(np.float64)).T)
    err = np.abs(logits.astype(np.float64) - exact)
    assert np.all(err <= bound), f"score error {err.max()} above the FP32 bound"
    want_ids, want_p = oracle.router_topk(logits, k, renormalize=renorm)
    assert np.array_equal(ids, want_ids), "top-k ids"
    n = k if renorm else w.shape[0]
    rel = np.abs(probs.astype(np.float64) - want_p) / want_p
    assert rel.max() <= (n + 8) * U, f"probability rel error {rel.max()}"
    return logits, ids, probs, float(err.max()), float(rel.max())


@pytest.mark.parametrize("renorm", [True, False])
@pytest.mark.parametrize("case", ["tiny", "qwen3"])
def test_router_parity(gpu, case, renorm):
    m, dev = gpu
    wl = W.tiny(seed=0) if case == "tiny" else W.qwen3(seed=2, T=4096)
    s = wl.shape
    w = _router_weights(s.E, s.H, 21)
    _, _, _, e_l, e_p = _check(m, dev, wl.x, w, s.K, renorm)
    print(f"  {case} renorm={renorm}: T={s.T} E={s.E} K={s.K}, max score error {e_l:.3g}, max prob rel {e_p:.3g}")


@pytest.mark.parametrize("T,H,E,K", [(33, 144, 50, 7), (5, 2048, 1024, 32), (70, 64, 3, 3),
                                     (33, 144, 200, 8), (70, 256, 256, 8), (5, 144, 257, 8),
                                     (40, 128, 129, 8), (9, 128, 255, 32)])
def test_router_ragged_shapes(gpu, T, H, E, K):
    """Expert counts that are not multiples of 32 or 64, the largest E and K, a
    token count with a partial 32-token tile, H not a multiple of 64; both
    top-k paths: rank counting (E <= 256, including 129..256 with four keys per
    lane and the E = 256 edge) and the rounds of wave-wide maxima (E = 257 and
    1024)."""
    m, dev = gpu
    rng = np.random.default_rng(E)
    x = W.f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
    w = _router_weights(E, H, 24)
    for renorm in (True, False):
        _check(m, dev, x, w, K, renorm)


def test_router_batch_invariance(gpu):
    m, dev = gpu
    wl = W.qwen3(seed=2, T=4096)
    s = wl.shape
    w = to_dev(_router_weights(s.E, s.H, 22), dev)
    x = to_dev(wl.x, dev)
    full = [to_host(a) for a in m.router_topk(x, w, s.K)]
    rng = np.random.default_rng(9)
    for T in (1, 7, 37, 100):
        rows = rng.choice(s.T, size=T, replace=False)
        part = [to_host(a) for a in m.router_topk(x[rows.tolist()].contiguous(), w, s.K)]
        for a, b, name in zip(part, full, ("scores", "ids", "probs")):
            assert np.array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                  (b[rows].view(np.uint32) if b.dtype == np.float32 else b[rows])), f"{name}, T={T}"


def test_router_out_buffers_are_checked(gpu):
    """Caller-provided output tensors of the wrong shape, dtype or layout raise
    before the kernel is launched."""
    import torch
    m, dev = gpu
    T, H, E, K = 8, 128, 16, 4
    x = to_dev(W.f32_to_bf16_bits(np.ones((T, H), np.float32)), dev)
    w = to_dev(_router_weights(E, H, 25), dev)
    good = (torch.empty((T, E), dtype=torch.float32, device=dev), torch.empty((T, K), dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.float32, device=dev))
    m.router_topk(x, w, K, out=good)
    for bad in ((good[0][:, :E - 1], good[1], good[2]), (good[0], good[1].float(), good[2]),
                (good[0], good[1], torch.empty((K, T), dtype=torch.float32, device=dev).t()),
                (good[0].cpu(), good[1], good[2])):
        with pytest.raises(ValueError):
            m.router_topk(x, w, K, out=bad)


@pytest.mark.parametrize("E", [64, 256])
def test_router_ties_go_to_the_lower_id(gpu, E):
    m, dev = gpu
    H, K = 256, 6
    w = _router_weights(E, H, 23)
    w[9] = w[5]      # experts 5 and 9 always score the same
    w[40] = w[12]    # and 12 and 40
    rng = np.random.default_rng(4)
    x = W.f32_to_bf16_bits(rng.standard_normal((300, H)).astype(np.float32))
    x[0] = 0          # a zero token: every score is 0
    logits, ids, probs, _, _ = _check(m, dev, x, w, K, True)
    assert ids[0].tolist() == list(range(K)) and np.all(probs[0] == np.float32(1.0 / K))
    for t in range(1, x.shape[0]):
        sel = ids[t].tolist()
        for a, b in ((5, 9), (12, 40)):
            if b in sel:
                assert a in sel and sel.index(a) == sel.index(b) - 1, f"token {t}: tie {a}/{b} order {sel}"
    hit = sum(5 in ids[t] for t in range(1, x.shape[0]))
    assert hit > 0
    print(f"  tied pair (5, 9) selected for {hit} tokens, always 5 first")
