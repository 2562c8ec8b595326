"""The allocation-free forward (nvfp4moe_moe_expert_forward_noalloc) against
the workspace forward (nvfp4moe_moe_expert_forward) through the C ABI: the
same kernels on the same inputs, so every output bit must agree.  Two calls
in a row on each layer shape, the second with fewer tokens (the static
scratch keeps the first call's contents); the device error word it copies
out; a token count whose intermediates exceed the scratch is refused before
any launch."""
import ctypes

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


def _layer(m, dev, wl, max_tokens):
    s = wl.shape
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, max_tokens)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    return cfg, qw


@pytest.mark.parametrize("case", ["tiny", "qwen3"])
def test_noalloc_equals_workspace_forward(gpu, case):
    import torch
    m, dev = gpu
    wl = W.tiny(seed=0) if case == "tiny" else W.qwen3(seed=2, T=512)
    sizes = (64, 17) if case == "tiny" else (512, 40)
    cfg, qw = _layer(m, dev, wl, max_tokens=wl.shape.T)
    ws = m.alloc_workspace(cfg, dev)
    err = torch.full((1,), -1, dtype=torch.int32, device=dev)
    for T in sizes:
        x, ids, probs = to_dev(wl.x[:T], dev), to_dev(wl.ids[:T], dev), to_dev(wl.probs[:T], dev)
        want = m.moe_expert_forward(cfg, x, ids, probs, qw, ws)
        got = m.moe_expert_forward_noalloc(cfg, x, ids, probs, qw, err_word=err)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"{case} T={T}"
        assert int(err.item()) == 0
        err.fill_(-1)
    print(f"  {case}: T = {sizes} bitwise equal to the workspace forward")


def test_noalloc_error_word_and_limits(gpu):
    import torch
    m, dev = gpu
    wl = W.tiny(seed=0)
    cfg, qw = _layer(m, dev, wl, max_tokens=64)
    ids = wl.ids.copy()
    ids[3, 1] = 8  # out of range: reported, nothing faults
    err = torch.zeros((1,), dtype=torch.int32, device=dev)
    m.moe_expert_forward_noalloc(cfg, to_dev(wl.x, dev), to_dev(ids, dev), to_dev(wl.probs, dev), qw, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & 1
    # the Qwen3-30B-A3B shape with 4096 tokens needs about 270 MB of intermediates
    big = W.qwen3(seed=2, T=4096)
    s = big.shape
    cfg_b = m.make_config(s.H, s.I, s.E, s.K, s.T)
    assert m.workspace_bytes(cfg_b) > m.NOALLOC_SCRATCH_BYTES
    qw_b = m.QuantWeights(cfg_b, dev)
    out = torch.empty((s.T, s.H), dtype=torch.int16, device=dev)
    st = m.lib().nvfp4moe_moe_expert_forward_noalloc(ctypes.byref(cfg_b), ctypes.c_void_p(out.data_ptr()), s.T,
                                                     ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                                                     ctypes.byref(qw_b.W1q), ctypes.byref(qw_b.W2q),
                                                     ctypes.c_void_p(out.data_ptr()), None, None)
    assert m.STATUS[st] == "NVFP4_E_SCRATCH"
    assert "scratch" in m.status_str(st)
    # T above max_tokens
    st = m.lib().nvfp4moe_moe_expert_forward_noalloc(ctypes.byref(cfg), None, 65, None, None, ctypes.byref(qw.W1q),
                                                     ctypes.byref(qw.W2q), None, None, None)
    assert m.STATUS[st] == "NVFP4_E_CAPACITY"
    # T = 0 is a no-op
    st = m.lib().nvfp4moe_moe_expert_forward_noalloc(ctypes.byref(cfg), None, 0, None, None, ctypes.byref(qw.W1q),
                                                     ctypes.byref(qw.W2q), None, None, None)
    assert st == 0
