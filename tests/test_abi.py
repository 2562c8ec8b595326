"""The C-ABI library: it loads, exports every function include/nvfp4moe.h
declares, and rejects bad arguments on the host before launching anything.
No GPU needed (only host-side paths are called)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")


@pytest.fixture(scope="module")
def m():
    import nvfp4_moe_expert_sort_amd as m
    if not os.path.exists(m.LIB_PATH):
        from nvfp4_moe_expert_sort_amd import build
        build.build()
    m.lib()
    return m


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"NVFP4MOE_API\s+[\w\s\*]+?\b(nvfp4\w+)\s*\(", src)))


def test_header_declares_the_documented_entry_points():
    names = _declared()
    for n in ("nvfp4_quantize", "nvfp4moe_moe_expert_forward", "nvfp4moe_selftest_batch_invariance"):
        assert n in names


def test_library_exports_every_declared_symbol(m):
    lib = m.lib()
    names = _declared()
    assert sorted(m.EXPORTS) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(m):
    lib = m.lib()
    assert lib.nvfp4_status_str(0) == b"ok"
    assert lib.nvfp4_status_str(4) == b"workspace too small"
    assert lib.nvfp4_status_str(99) == b"unknown status"


def _cfg(m, **kw):
    base = dict(hidden=2048, inter=768, n_experts=128, top_k=8, max_tokens=4096, scale_round=0)
    base.update(kw)
    return m.make_config(**base)


def test_workspace_bytes_depend_on_config_only(m):
    a = m.workspace_bytes(_cfg(m))
    assert a > 0 and a % 256 == 0
    assert m.workspace_bytes(_cfg(m, max_tokens=8192)) > a
    lay = m.workspace_layout(_cfg(m))
    assert lay.m_align == 32 and lay.n_part == 768 // 32
    assert lay.rows_cap >= 4096 * 8 + 128 * 31 and lay.rows_cap % 32 == 0
    offs = [lay.err, lay.expert_count, lay.expert_off, lay.pair2row, lay.row2pair, lay.a1_codes, lay.a1_scales,
            lay.a1_g, lay.h, lay.amax2_part, lay.a2_codes, lay.a2_scales, lay.a2_g, lay.y2]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs) and offs[-1] < a


@pytest.mark.parametrize("bad", [dict(hidden=2000), dict(inter=100), dict(n_experts=0), dict(n_experts=2048),
                                 dict(top_k=0), dict(top_k=33), dict(top_k=9, n_experts=8), dict(max_tokens=-1),
                                 dict(scale_round=2)])
def test_invalid_configs_are_rejected(m, bad):
    cfg = _cfg(m, **bad)
    lib = m.lib()
    assert lib.nvfp4moe_workspace_bytes(ctypes.byref(cfg)) == 0
    assert lib.nvfp4moe_weight_bytes(ctypes.byref(cfg), 1) == 0
    st = lib.nvfp4moe_moe_expert_forward(ctypes.byref(cfg), None, 1, None, None, None, None, None, None, 0, None)
    assert st == 2


def test_forward_host_validation(m):
    lib = m.lib()
    cfg = _cfg(m, max_tokens=64)
    E, H, I = 128, 2048, 768
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    W1 = m.QTensor(0x1000, 0x1000, 0x1000, E, 2 * I, H, m.LAYOUT_GEMM)
    W2 = m.QTensor(0x1000, 0x1000, 0x1000, E, H, I, m.LAYOUT_GEMM)
    need = m.workspace_bytes(cfg)
    # the standard forward and the one that quantizes X inside FC1 share the checks
    for f in (lib.nvfp4moe_moe_expert_forward, lib.nvfp4moe_moe_expert_forward_online):
        # null config / weights / workspace
        assert f(None, fake, 1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake, fake, need, None) == 1
        assert f(ctypes.byref(cfg), fake, 1, fake, fake, None, ctypes.byref(W2), fake, fake, need, None) == 1
        assert f(ctypes.byref(cfg), fake, 1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake, None, need, None) == 1
        # capacity and negative T
        assert f(ctypes.byref(cfg), fake, 65, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake, fake, need, None) == 5
        assert f(ctypes.byref(cfg), fake, -1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake, fake, need, None) == 2
        # undersized workspace
        assert f(ctypes.byref(cfg), fake, 1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake, fake, need - 1,
                 None) == 4
        # weight tensor of the wrong shape or layout
        bad = m.QTensor(0x1000, 0x1000, 0x1000, E, I, H, m.LAYOUT_GEMM)
        assert f(ctypes.byref(cfg), fake, 1, fake, fake, ctypes.byref(bad), ctypes.byref(W2), fake, fake, need, None) == 2
        bad = m.QTensor(0x1000, 0x1000, 0x1000, E, 2 * I, H, m.LAYOUT_LOGICAL)
        assert f(ctypes.byref(cfg), fake, 1, fake, fake, ctypes.byref(bad), ctypes.byref(W2), fake, fake, need, None) == 2
        # misaligned workspace and activations
        assert f(ctypes.byref(cfg), fake, 1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake,
                 ctypes.c_void_p(0x1010), need, None) == 3
        assert f(ctypes.byref(cfg), ctypes.c_void_p(0x1002), 1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake,
                 fake, need, None) == 3
        # null activations with T > 0
        assert f(ctypes.byref(cfg), None, 1, fake, fake, ctypes.byref(W1), ctypes.byref(W2), fake, fake, need, None) == 1
        # T == 0 is a no-op that launches nothing
        assert f(ctypes.byref(cfg), None, 0, None, None, ctypes.byref(W1), ctypes.byref(W2), None, fake, need, None) == 0


def test_backward_host_validation(m):
    """nvfp4moe_moe_expert_backward rejects bad arguments on the host, before
    launching anything, with the forward's error codes."""
    lib = m.lib()
    cfg = _cfg(m, max_tokens=64)
    rows = int(m.workspace_layout(cfg).rows_cap)
    fwd = m.workspace_bytes(cfg)
    need = lib.nvfp4moe_backward_workspace_bytes(ctypes.byref(cfg))
    assert need > 0 and need % 256 == 0
    assert lib.nvfp4moe_backward_workspace_bytes(ctypes.byref(_cfg(m, max_tokens=128))) > need
    assert lib.nvfp4moe_backward_workspace_bytes(ctypes.byref(_cfg(m, hidden=100))) == 0
    f = lib.nvfp4moe_moe_expert_backward
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first

    def call(cfgp=ctypes.byref(cfg), x=fake, T=1, y1_rows=rows, fw=fake, fw_bytes=fwd, ws=fake, ws_bytes=need,
             dprobs=fake, dout=fake):
        return f(cfgp, x, T, fake, fake, fake, y1_rows, fw, fw_bytes, dout, fake, dprobs, fake, fake, ws, ws_bytes,
                 None)

    assert call(cfgp=None) == 1                             # null config
    assert call(cfgp=ctypes.byref(_cfg(m, hidden=100))) == 2  # bad config
    assert call(T=-1) == 2 and call(T=65) == 5              # negative T, T past max_tokens
    assert call(y1_rows=rows - 1) == 2                      # y1 shorter than the sorted rows
    assert call(fw=None) == 1 and call(ws=None) == 1        # null workspaces
    assert call(fw_bytes=fwd - 1) == 4 and call(ws_bytes=need - 1) == 4
    assert call(fw=ctypes.c_void_p(0x1010)) == 3 and call(ws=ctypes.c_void_p(0x1080)) == 3
    assert call(T=0, x=None, dout=None, dprobs=None) == 0   # T == 0 launches nothing
    assert call(x=None) == 1 and call(dout=None) == 1       # null tensors with T > 0
    assert call(x=ctypes.c_void_p(0x1002)) == 3 and call(dprobs=ctypes.c_void_p(0x1002)) == 3


def test_masked_layout_sizes_and_host_validation(m):
    """Masked fixed-capacity layout: E chunks of `capacity` rows (a positive
    multiple of 32), checked on the host before anything is launched."""
    lib = m.lib()
    cfg = _cfg(m, max_tokens=64)
    E, H, I = 128, 2048, 768
    for bad in (0, -32, 16, 33, 1 << 23):  # 1 << 23 rows per expert: E * capacity >= 2**30
        assert lib.nvfp4moe_workspace_bytes_masked(ctypes.byref(cfg), bad) == 0
        lay = m.WsLayout()
        assert lib.nvfp4moe_workspace_layout_masked(ctypes.byref(cfg), bad, ctypes.byref(lay)) == 2
    lay = m.workspace_layout_masked(cfg, 96)
    assert lay.rows_cap == E * 96 and lay.m_align == 32
    offs = [lay.err, lay.expert_count, lay.expert_off, lay.pair2row, lay.row2pair, lay.a1_codes, lay.a1_scales,
            lay.a1_g, lay.h, lay.amax2_part, lay.a2_codes, lay.a2_scales, lay.a2_g, lay.y2]
    need = m.workspace_bytes_masked(cfg, 96)
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs) and offs[-1] < need
    # the chunks, not max_tokens, size the row buffers
    assert m.workspace_bytes_masked(cfg, 192) > need
    assert m.workspace_layout_masked(_cfg(m, max_tokens=4096), 96).rows_cap == E * 96
    f = lib.nvfp4moe_moe_expert_forward_masked
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    W1 = m.QTensor(0x1000, 0x1000, 0x1000, E, 2 * I, H, m.LAYOUT_GEMM)
    W2 = m.QTensor(0x1000, 0x1000, 0x1000, E, H, I, m.LAYOUT_GEMM)
    args = lambda cap, T, ws_bytes: (ctypes.byref(cfg), cap, fake, T, fake, fake, ctypes.byref(W1), ctypes.byref(W2),
                                     fake, fake, ws_bytes, None)
    assert f(*args(48, 1, need)) == 2     # capacity not a multiple of 32
    assert f(*args(96, 65, need)) == 5    # T > max_tokens
    assert f(*args(96, 1, need - 1)) == 4  # workspace sized for this capacity
    assert f(*args(192, 1, need)) == 4    # a larger capacity needs a larger workspace
    assert f(*args(96, 0, need)) == 0     # T == 0: no-op


def test_router_host_validation(m):
    f = m.lib().nvfp4moe_router_topk
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    ok = dict(T=4, H=256, E=64, K=8, renorm=1)

    def call(**kw):
        a = dict(ok, **kw)
        return f(fake, a["T"], a["H"], fake, a["E"], a["K"], a["renorm"], fake, fake, fake, None)
    assert call(H=200) == 2 and call(H=0) == 2          # H % 16
    assert call(E=0) == 2 and call(E=2048) == 2         # 1 <= E <= 1024
    assert call(K=0) == 2 and call(K=65) == 2 and call(E=4, K=5) == 2 and call(E=64, K=33) == 2
    assert call(T=-1) == 2
    assert call(renorm=2) == 9
    assert call(T=0) == 0                               # no-op
    assert f(None, 4, 256, fake, 64, 8, 1, fake, fake, fake, None) == 1
    assert f(ctypes.c_void_p(0x1004), 4, 256, fake, 64, 8, 1, fake, fake, fake, None) == 3


def test_quantize_host_validation(m):
    q = m.lib().nvfp4_quantize
    fake = ctypes.c_void_p(0x1000)
    assert q(fake, 4, 64, 64, fake, fake, fake, 2, 0, None) == 9        # bad layout
    assert q(fake, 4, 64, 64, fake, fake, fake, 0, 5, None) == 9        # bad rounding
    assert q(fake, 4, 40, 64, fake, fake, fake, 0, 0, None) == 2        # cols % 16
    assert q(fake, 4, 64, 32, fake, fake, fake, 0, 0, None) == 2        # ld < cols
    assert q(fake, 4, 128, 128, fake, fake, fake, 1, 0, None) == 2      # GEMM layout needs rows % 32
    assert q(fake, 32, 64, 64, fake, fake, fake, 1, 0, None) == 2       # GEMM layout needs cols % 128
    assert q(None, 4, 64, 64, fake, fake, fake, 0, 0, None) == 1
    assert q(ctypes.c_void_p(0x1002), 4, 64, 64, fake, fake, fake, 0, 0, None) == 3
    assert q(None, 0, 64, 64, None, None, None, 0, 0, None) == 0        # empty is a no-op


def test_linear_host_validation(m):
    lib = m.lib()
    fake = ctypes.c_void_p(0x1000)
    Wq = m.QTensor(0x1000, 0x1000, 0x1000, 1, 1536, 2048, m.LAYOUT_GEMM)
    need = lib.nvfp4_linear_workspace_bytes(4096, 2048)
    assert need > 0 and lib.nvfp4_linear_workspace_bytes(4, 100) == 0
    assert lib.nvfp4_linear(fake, 4096, 2048, ctypes.byref(Wq), fake, 0, fake, need - 1, None) == 4
    assert lib.nvfp4_linear(fake, 4096, 1024, ctypes.byref(Wq), fake, 0, fake, need, None) == 2
    assert lib.nvfp4_linear(fake, 4096, 2048, None, fake, 0, fake, need, None) == 1
    assert lib.nvfp4_linear(fake, 4096, 2048, ctypes.byref(Wq), fake, 3, fake, need, None) == 9


def test_selftest_argument_checks(m):
    lib = m.lib()
    cfg = _cfg(m, max_tokens=64)
    W = m.QTensor(0x1000, 0x1000, 0x1000, 128, 1536, 2048, m.LAYOUT_GEMM)
    rep = (ctypes.c_int64 * 4)()
    assert lib.nvfp4moe_selftest_batch_invariance(ctypes.byref(cfg), ctypes.byref(W), ctypes.byref(W), 1, 0, 4, 0,
                                                  rep, None) == 2
    assert lib.nvfp4moe_selftest_batch_invariance(ctypes.byref(cfg), ctypes.byref(W), ctypes.byref(W), 1, 4, 65,
                                                  0, rep, None) == 5
