"""MI355X (gfx950) NVFP4 MoE expert forward -- Python binding of libnvfp4moe.so.

Argument marshalling only: every step of the path runs in the HIP library
(``include/nvfp4moe.h`` documents each entry point).  PyTorch supplies device
memory and the current stream.  The binding fails loudly when the library is
missing: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libnvfp4moe.so")

NVFP4_OK = 0
STATUS = {0: "NVFP4_OK", 1: "NVFP4_E_NULL", 2: "NVFP4_E_SHAPE", 3: "NVFP4_E_ALIGN", 4: "NVFP4_E_WORKSPACE",
          5: "NVFP4_E_CAPACITY", 6: "NVFP4_E_HIP", 7: "NVFP4_E_MISMATCH", 8: "NVFP4_E_DEVICE", 9: "NVFP4_E_ARG",
          10: "NVFP4_E_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 64 << 20
SCALE_RU = 0
SCALE_RNE = 1
LAYOUT_LOGICAL = 0
LAYOUT_GEMM = 1

# Every function the C header declares (checked against the header by the tests).
EXPORTS = ["nvfp4_status_str", "nvfp4_quantize", "nvfp4moe_weight_bytes", "nvfp4moe_quantize_weights",
           "nvfp4moe_workspace_bytes", "nvfp4moe_moe_expert_forward", "nvfp4moe_moe_expert_forward_events",
           "nvfp4moe_device_error",
           "nvfp4moe_workspace_layout", "nvfp4moe_workspace_bytes_masked", "nvfp4moe_workspace_layout_masked",
           "nvfp4moe_moe_expert_forward_masked", "nvfp4moe_moe_expert_forward_unfused",
           "nvfp4moe_moe_expert_forward_noalloc", "nvfp4moe_backward_workspace_bytes", "nvfp4moe_moe_expert_backward",
           "nvfp4moe_moe_expert_forward_w4a16", "nvfp4moe_moe_expert_forward_online", "nvfp4moe_router_topk", "nvfp4_linear_workspace_bytes", "nvfp4_linear",
           "nvfp4moe_selftest_batch_invariance"]


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("scale_round", ctypes.c_int32)]


class QTensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("g", ctypes.c_void_p),
                ("n_mats", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32),
                ("layout", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("err", "expert_count", "expert_off", "pair2row", "row2pair", "a1_codes", "a1_scales", "a1_g", "h",
                 "amax2_part", "a2_codes", "a2_scales", "a2_g", "y2")] + \
               [("rows_cap", ctypes.c_int64), ("m_align", ctypes.c_int32), ("n_part", ctypes.c_int32)]


_lib = None


def lib():
    """Load libnvfp4moe.so (built by ``build.build()``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cfgp, qtp = ctypes.POINTER(Config), ctypes.POINTER(QTensor)
    sig = {
        "nvfp4_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "nvfp4_quantize": (ctypes.c_int, [vp, i64, i64, i64, vp, vp, vp, i32, i32, vp]),
        "nvfp4moe_weight_bytes": (sz, [cfgp, i32]),
        "nvfp4moe_quantize_weights": (ctypes.c_int, [cfgp, vp, vp, qtp, qtp, vp]),
        "nvfp4moe_workspace_bytes": (sz, [cfgp]),
        "nvfp4moe_moe_expert_forward": (ctypes.c_int, [cfgp, vp, i32, vp, vp, qtp, qtp, vp, vp, sz, vp]),
        "nvfp4moe_moe_expert_forward_events": (ctypes.c_int, [cfgp, vp, i32, vp, vp, qtp, qtp, vp, vp, sz,
                                                               ctypes.POINTER(vp), vp]),
        "nvfp4moe_device_error": (ctypes.c_int, [cfgp, vp, ctypes.POINTER(i32), vp]),
        "nvfp4moe_workspace_layout": (ctypes.c_int, [cfgp, ctypes.POINTER(WsLayout)]),
        "nvfp4moe_workspace_bytes_masked": (sz, [cfgp, i32]),
        "nvfp4moe_workspace_layout_masked": (ctypes.c_int, [cfgp, i32, ctypes.POINTER(WsLayout)]),
        "nvfp4moe_moe_expert_forward_masked": (ctypes.c_int, [cfgp, i32, vp, i32, vp, vp, qtp, qtp, vp, vp, sz, vp]),
        "nvfp4moe_moe_expert_forward_w4a16": (ctypes.c_int, [cfgp, vp, i32, vp, vp, qtp, qtp, vp, vp, sz, vp]),
        "nvfp4moe_moe_expert_forward_online": (ctypes.c_int, [cfgp, vp, i32, vp, vp, qtp, qtp, vp, vp, sz, vp]),
        "nvfp4moe_backward_workspace_bytes": (sz, [cfgp]),
        "nvfp4moe_moe_expert_backward": (ctypes.c_int, [cfgp, vp, i32, vp, vp, vp, i64, vp, sz, vp, vp, vp, vp, vp, vp,
                                                         sz, vp]),
        "nvfp4moe_moe_expert_forward_noalloc": (ctypes.c_int, [cfgp, vp, i32, vp, vp, qtp, qtp, vp, vp, vp]),
        "nvfp4moe_moe_expert_forward_unfused": (ctypes.c_int, [cfgp, vp, i32, vp, vp, qtp, qtp, vp, vp, i64, vp, sz,
                                                                vp]),
        "nvfp4moe_router_topk": (ctypes.c_int, [vp, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp]),
        "nvfp4_linear_workspace_bytes": (sz, [i64, i64]),
        "nvfp4_linear": (ctypes.c_int, [vp, i64, i64, qtp, vp, i32, vp, sz, vp]),
        "nvfp4moe_selftest_batch_invariance": (ctypes.c_int, [cfgp, qtp, qtp, ctypes.c_uint64, i32, i32, i32,
                                                              ctypes.POINTER(i64), vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int, where: str):
    if status != NVFP4_OK:
        raise Nvfp4Error(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_config(hidden, inter, n_experts, top_k, max_tokens, scale_round=SCALE_RU) -> Config:
    return Config(hidden, inter, n_experts, top_k, max_tokens, scale_round)


def status_str(status: int) -> str:
    return lib().nvfp4_status_str(status).decode()


# --- quantizer ------------------------------------------------------------------------------------

def quantize(x, layout: int = LAYOUT_LOGICAL, scale_round: int = SCALE_RU, stream=None):
    """nvfp4_quantize over a [rows, cols] BF16 CUDA tensor (uint16/int16/bfloat16 storage).

    Returns (codes [rows, cols/2] uint8, scales [rows, cols/16] uint8, g [rows] float32)."""
    import torch
    rows, cols = x.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty((rows,), dtype=torch.float32, device=x.device)
    st = lib().nvfp4_quantize(_ptr(x), rows, cols, x.stride(0), _ptr(codes), _ptr(scales), _ptr(g), layout,
                              scale_round, _stream(stream))
    _check(st, "nvfp4_quantize")
    return codes, scales, g


def qtensor(codes, scales, g, n_mats, rows, cols, layout=LAYOUT_GEMM) -> QTensor:
    return QTensor(codes.data_ptr(), scales.data_ptr(), g.data_ptr(), n_mats, rows, cols, layout)


class QuantWeights:
    """Caller-owned GEMM-layout buffers for W1 [E, 2I, H] and W2 [E, H, I]."""

    def __init__(self, cfg: Config, device="cuda"):
        import torch
        E, H, I = cfg.n_experts, cfg.hidden, cfg.inter
        self.cfg = cfg
        self.w1_codes = torch.empty((E * 2 * I, H // 2), dtype=torch.uint8, device=device)
        self.w1_scales = torch.empty((E * 2 * I, H // 16), dtype=torch.uint8, device=device)
        self.w1_g = torch.empty((E * 2 * I,), dtype=torch.float32, device=device)
        self.w2_codes = torch.empty((E * H, I // 2), dtype=torch.uint8, device=device)
        self.w2_scales = torch.empty((E * H, I // 16), dtype=torch.uint8, device=device)
        self.w2_g = torch.empty((E * H,), dtype=torch.float32, device=device)
        self.W1q = qtensor(self.w1_codes, self.w1_scales, self.w1_g, E, 2 * I, H)
        self.W2q = qtensor(self.w2_codes, self.w2_scales, self.w2_g, E, H, I)

    def quantize_from(self, w1, w2, stream=None):
        """nvfp4moe_quantize_weights: BF16 w1 [E,2I,H], w2 [E,H,I] -> these buffers, in place."""
        st = lib().nvfp4moe_quantize_weights(ctypes.byref(self.cfg), _ptr(w1), _ptr(w2), ctypes.byref(self.W1q),
                                             ctypes.byref(self.W2q), _stream(stream))
        _check(st, "nvfp4moe_quantize_weights")
        return self


def workspace_bytes(cfg: Config) -> int:
    n = lib().nvfp4moe_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise Nvfp4Error(2, "nvfp4moe_workspace_bytes")
    return n


def workspace_layout(cfg: Config) -> WsLayout:
    out = WsLayout()
    _check(lib().nvfp4moe_workspace_layout(ctypes.byref(cfg), ctypes.byref(out)), "nvfp4moe_workspace_layout")
    return out


def alloc_workspace(cfg: Config, device="cuda"):
    import torch
    return torch.empty((workspace_bytes(cfg),), dtype=torch.uint8, device=device)


def workspace_bytes_masked(cfg: Config, capacity: int) -> int:
    n = lib().nvfp4moe_workspace_bytes_masked(ctypes.byref(cfg), capacity)
    if n == 0:
        raise Nvfp4Error(2, "nvfp4moe_workspace_bytes_masked")
    return n


def workspace_layout_masked(cfg: Config, capacity: int) -> WsLayout:
    out = WsLayout()
    _check(lib().nvfp4moe_workspace_layout_masked(ctypes.byref(cfg), capacity, ctypes.byref(out)),
           "nvfp4moe_workspace_layout_masked")
    return out


def alloc_workspace_masked(cfg: Config, capacity: int, device="cuda"):
    import torch
    return torch.empty((workspace_bytes_masked(cfg, capacity),), dtype=torch.uint8, device=device)


def moe_expert_forward_masked(cfg: Config, capacity: int, x, ids, probs, weights: QuantWeights, workspace, out=None,
                              stream=None):
    """nvfp4moe_moe_expert_forward_masked: as moe_expert_forward, with expert e's rows in the fixed chunk
    [e*capacity, (e+1)*capacity) of the workspace's sorted buffers."""
    import torch
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    st = lib().nvfp4moe_moe_expert_forward_masked(ctypes.byref(cfg), capacity, _ptr(x), T, _ptr(ids), _ptr(probs),
                                                  ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward_masked")
    return out


def moe_expert_forward_w4a16(cfg: Config, x, ids, probs, weights: QuantWeights, workspace, out=None, stream=None):
    """nvfp4moe_moe_expert_forward_w4a16: as moe_expert_forward with BF16 activations (NVFP4 weights only)."""
    import torch
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    st = lib().nvfp4moe_moe_expert_forward_w4a16(ctypes.byref(cfg), _ptr(x), T, _ptr(ids), _ptr(probs),
                                                 ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                                 _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward_w4a16")
    return out


def moe_expert_forward_online(cfg: Config, x, ids, probs, weights: QuantWeights, workspace, out=None, stream=None):
    """nvfp4moe_moe_expert_forward_online: moe_expert_forward with X quantized inside FC1 (same output bits)."""
    import torch
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    st = lib().nvfp4moe_moe_expert_forward_online(ctypes.byref(cfg), _ptr(x), T, _ptr(ids), _ptr(probs),
                                                  ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward_online")
    return out


def moe_expert_backward(cfg: Config, x, w1, w2, y1, fwd_workspace, dout, stream=None):
    """nvfp4moe_moe_expert_backward after moe_expert_forward_unfused(cfg, x, ...) filled fwd_workspace and
    y1: BF16 w1 [E, 2I, H], w2 [E, H, I], dout [T, H] -> (dx [T, H] BF16, dprobs [T, K] f32,
    dw1 [E, 2I, H] f32, dw2 [E, H, I] f32)."""
    import torch
    T = x.shape[0]
    E, H, I, K = cfg.n_experts, cfg.hidden, cfg.inter, cfg.top_k
    dev = x.device
    dx = torch.empty((T, H), dtype=x.dtype, device=dev)
    dprobs = torch.empty((T, K), dtype=torch.float32, device=dev)
    dw1 = torch.empty((E, 2 * I, H), dtype=torch.float32, device=dev)
    dw2 = torch.empty((E, H, I), dtype=torch.float32, device=dev)
    n = lib().nvfp4moe_backward_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise Nvfp4Error(2, "nvfp4moe_backward_workspace_bytes")
    ws = torch.empty((n,), dtype=torch.uint8, device=dev)
    st = lib().nvfp4moe_moe_expert_backward(ctypes.byref(cfg), _ptr(x), T, _ptr(w1), _ptr(w2), _ptr(y1), y1.shape[0],
                                            _ptr(fwd_workspace), fwd_workspace.numel(), _ptr(dout), _ptr(dx),
                                            _ptr(dprobs), _ptr(dw1), _ptr(dw2), _ptr(ws), n, _stream(stream))
    _check(st, "nvfp4moe_moe_expert_backward")
    return dx, dprobs, dw1, dw2, ws


def moe_expert_forward_noalloc(cfg: Config, x, ids, probs, weights: QuantWeights, out=None, err_word=None,
                               stream=None):
    """nvfp4moe_moe_expert_forward_noalloc: as moe_expert_forward, with the intermediates in the library's
    static per-GPU scratch (no workspace, no allocation by the library; `out` and `err_word`, a device
    int32 that receives the device error word, may be given preallocated)."""
    import torch
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    st = lib().nvfp4moe_moe_expert_forward_noalloc(ctypes.byref(cfg), _ptr(x), T, _ptr(ids), _ptr(probs),
                                                   ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                                   _ptr(err_word), _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward_noalloc")
    return out


def moe_expert_forward_unfused(cfg: Config, x, ids, probs, weights: QuantWeights, workspace, y1=None, out=None,
                               stream=None):
    """nvfp4moe_moe_expert_forward_unfused: the forward with FC1 writing y1 [rows_cap, 2I] BF16 and the
    SwiGLU producer as a separate kernel.  Returns (out, y1)."""
    import torch
    T = x.shape[0]
    rows = workspace_layout(cfg).rows_cap
    if out is None:
        out = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    if y1 is None:
        y1 = torch.empty((rows, 2 * cfg.inter), dtype=x.dtype, device=x.device)
    st = lib().nvfp4moe_moe_expert_forward_unfused(ctypes.byref(cfg), _ptr(x), T, _ptr(ids), _ptr(probs),
                                                   ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                                   _ptr(y1), y1.shape[0], _ptr(workspace), workspace.numel(),
                                                   _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward_unfused")
    return out, y1


def moe_expert_forward(cfg: Config, x, ids, probs, weights: QuantWeights, workspace, out=None, stream=None):
    """nvfp4moe_moe_expert_forward: x [T,H] BF16, ids [T,K] int32, probs [T,K] float32 -> out [T,H] BF16."""
    import torch
    T = x.shape[0]
    if out is None:
        out = torch.empty((T, cfg.hidden), dtype=x.dtype, device=x.device)
    st = lib().nvfp4moe_moe_expert_forward(ctypes.byref(cfg), _ptr(x), T, _ptr(ids), _ptr(probs),
                                           ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                           _ptr(workspace), workspace.numel(), _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward")
    return out


N_STAGE_EVENTS = 6
STAGES = ["sort+quantize X", "FC1 + SwiGLU producer", "quantize h", "FC2", "combine"]


def moe_expert_forward_events(cfg: Config, x, ids, probs, weights: QuantWeights, workspace, events, out,
                              stream=None):
    """nvfp4moe_moe_expert_forward_events: as moe_expert_forward, recording the
    6 torch.cuda.Event objects in `events` at the stage boundaries on the stream."""
    arr = (ctypes.c_void_p * N_STAGE_EVENTS)(*[ctypes.c_void_p(e.cuda_event) for e in events])
    st = lib().nvfp4moe_moe_expert_forward_events(ctypes.byref(cfg), _ptr(x), x.shape[0], _ptr(ids), _ptr(probs),
                                                  ctypes.byref(weights.W1q), ctypes.byref(weights.W2q), _ptr(out),
                                                  _ptr(workspace), workspace.numel(), arr, _stream(stream))
    _check(st, "nvfp4moe_moe_expert_forward_events")
    return out


def device_error(cfg: Config, workspace, stream=None) -> int:
    code = ctypes.c_int32(0)
    _check(lib().nvfp4moe_device_error(ctypes.byref(cfg), _ptr(workspace), ctypes.byref(code), _stream(stream)),
           "nvfp4moe_device_error")
    return code.value


def router_topk(x, w_router, k: int, renormalize: bool = True, stream=None, out=None):
    """nvfp4moe_router_topk: x [T,H] BF16, w_router [E,H] BF16 -> (logits [T,E] f32, ids [T,k] int32,
    probs [T,k] f32); `out` may hold the three output tensors, preallocated."""
    import torch
    T, H = x.shape
    E = w_router.shape[0]
    if out is not None:
        logits, ids, probs = out
        for t, name, shape, dtype in ((logits, "logits", (T, E), torch.float32), (ids, "ids", (T, k), torch.int32),
                                      (probs, "probs", (T, k), torch.float32)):
            if tuple(t.shape) != shape or t.dtype != dtype or not t.is_contiguous() or t.device != x.device:
                raise ValueError(f"router_topk: out {name} must be a contiguous {dtype} tensor of shape {shape} "
                                 f"on {x.device}, got {tuple(t.shape)} {t.dtype} on {t.device}")
    else:
        logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
        ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
        probs = torch.empty((T, k), dtype=torch.float32, device=x.device)
    st = lib().nvfp4moe_router_topk(_ptr(x), T, H, _ptr(w_router), E, k, 1 if renormalize else 0, _ptr(logits),
                                    _ptr(ids), _ptr(probs), _stream(stream))
    _check(st, "nvfp4moe_router_topk")
    return logits, ids, probs


def linear_workspace_bytes(M: int, K: int) -> int:
    return lib().nvfp4_linear_workspace_bytes(M, K)


def linear(x, Wq: QTensor, workspace, scale_round: int = SCALE_RU, out=None, stream=None):
    """nvfp4_linear: x [M,K] BF16, Wq one GEMM-layout [N,K] matrix -> out [M,N] BF16."""
    import torch
    M, K = x.shape
    if out is None:
        out = torch.empty((M, Wq.rows), dtype=x.dtype, device=x.device)
    st = lib().nvfp4_linear(_ptr(x), M, K, ctypes.byref(Wq), _ptr(out), scale_round, _ptr(workspace),
                            workspace.numel(), _stream(stream))
    _check(st, "nvfp4_linear")
    return out


def selftest_batch_invariance(cfg: Config, weights: QuantWeights, seed: int, n_probe: int, max_decode_batch: int,
                              prefill_tokens: int, stream=None):
    """nvfp4moe_selftest_batch_invariance; returns (status, report dict)."""
    rep = (ctypes.c_int64 * 4)()
    st = lib().nvfp4moe_selftest_batch_invariance(ctypes.byref(cfg), ctypes.byref(weights.W1q),
                                                  ctypes.byref(weights.W2q), seed, n_probe, max_decode_batch,
                                                  prefill_tokens, rep, _stream(stream))
    return st, dict(n_compared=rep[0], n_mismatched=rep[1], first_bad_probe=rep[2], first_bad_batch=rep[3])
