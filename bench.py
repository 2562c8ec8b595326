"""Benchmark of the NVFP4 MoE expert forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one whole forward (sort + quantize X, FC1 with the SwiGLU producer,
quantize h, FC2, combine) over the Qwen3-30B-A3B-shaped layer with 4096
tokens (hidden 2048, 128 experts, top-8, expert intermediate 768; synthetic
seeded inputs and random weights, resident in HBM before timing).  W untimed
warm-up steps, then exactly K steps bracketed by device synchronisation.
Prints one JSON line.  The dominant kernel (FC1) is timed with HIP events
recorded on the forward's stream at its boundaries, in a pass of the same
forwards right after the timed region; the CPU oracle is timed on a bounded
sample on the host cores.

The secondary measurements (weight quantization, cold-cache forwards, the
dense linear, the skewed and W4A16 workloads, the masked layout, the BF16
backward, the router, decode sizes) run before the headline forwards.  They also bring the GPU
from idle to its steady clocks, which takes about 80 back-to-back forwards,
so the W warm-up steps and the K timed steps see the clocks of a layer that
runs continuously, whatever W is.
"""
from __future__ import annotations

import argparse
import glob
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense f16/bf16 MFMA
NOMINAL_SCLK_MHZ = 2400.0       # the clock that peak assumes
MFMA_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp4 MFMA (reported for context)
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The MI355X settles its clocks over the first ~80 back-to-back forwards
    # (~35 ms) after an idle period; the defaults warm past that and time the
    # steady state a layer sees when it runs continuously.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--tokens", type=int, default=4096)
    ap.add_argument("--cold-steps", type=int, default=50, help="extra forwards timed after a cache-evicting write")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-sized (T = 1, 8, 64) forwards")
    ap.add_argument("--no-w4a16", action="store_true", help="skip the W4A16 variant's forwards")
    ap.add_argument("--no-online", action="store_true",
                    help="skip the forward that quantizes X inside FC1 (secondary timing)")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense NVFP4 linear")
    ap.add_argument("--no-skewed", action="store_true", help="skip the skewed-routing T = 16384 forwards")
    ap.add_argument("--no-router", action="store_true", help="skip the on-device router (scores + top-k)")
    ap.add_argument("--no-masked", action="store_true", help="skip the masked fixed-capacity forward")
    ap.add_argument("--no-backward", action="store_true", help="skip the BF16 straight-through backward")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference dispatch for HBM byte counters)")
    ap.add_argument("--oracle-single-thread", action="store_true", help=argparse.SUPPRESS)
    return ap.parse_args()


def layer_bytes(T, H, E, K, I, counts):
    """Algorithmic HBM bytes of the layer as built (each intermediate written and read once)."""
    P = T * K
    qrow = lambda c: c // 2 + c // 16 + 4  # noqa: E731  packed codes + scales + g
    used = int((counts > 0).sum())
    w = used * (2 * I * qrow(H) + H * qrow(I))
    x_in, out = T * H * 2, T * H * 2
    a1, h, a2, y2 = P * qrow(H), P * I * 2, P * qrow(I), P * H * 2
    routing = T * K * 8
    return dict(weights=w, total=w + x_in + out + routing + 2 * (a1 + h + a2 + y2),
                fc1=a1 + used * 2 * I * qrow(H) + h, compulsory=w + x_in + out + routing)


PROFILE = os.path.join(ROOT, "profiles", "moe_forward_qwen3_T4096.md")
FC1_SOURCES = ["nvfp4_moe_expert_sort_amd/csrc/gemm.hip", "nvfp4_moe_expert_sort_amd/csrc/nvfp4_device.h",
               "nvfp4_moe_expert_sort_amd/csrc/nvfp4_kernels.h"]


def fc1_traffic_bytes():
    """HBM bytes per FC1 launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE summary,
    or None when the kernel sources changed since those counters were taken."""
    import hashlib
    try:
        text = open(PROFILE).read()
    except OSError:
        return None
    fields = dict(line.strip().split(": ", 1) for line in text.splitlines()
                  if line.strip().startswith(("fc1_traffic_bytes_per_launch:", "kernel_source_sha256:")))
    h = hashlib.sha256()
    for f in FC1_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_source_sha256") != h.hexdigest() or "fc1_traffic_bytes_per_launch" not in fields:
        return None
    return float(fields["fc1_traffic_bytes_per_launch"])


def sclk_path():
    """The sysfs file listing the GPU's shader clock levels, the current one
    marked with '*' (the first card that has one), or None."""
    for p in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            open(p).read()
            return p
        except OSError:
            continue
    return None


def read_sclk_mhz(path):
    for line in open(path).read().splitlines():
        if line.rstrip().endswith("*"):
            tok = [t for t in line.replace(":", " ").split() if t.lower().endswith("mhz")]
            if tok:
                return float(tok[0][:-3])
    return None


def observed_clock(run, seconds=0.15, interval_s=0.002):
    """Shader clock while `run()` keeps the GPU busy: pp_dpm_sclk read every
    2 ms from a host thread over about `seconds` of back-to-back forwards (a
    separate pass after the timed region, so the timing is not disturbed)."""
    path = sclk_path()
    if path is None:
        return None
    samples, stop = [], threading.Event()

    def sample():
        while not stop.is_set():
            v = read_sclk_mhz(path)
            if v is not None:
                samples.append(v)
            time.sleep(interval_s)

    th = threading.Thread(target=sample, daemon=True)
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        run()
    stop.set()
    th.join()
    if not samples:
        return None
    a = np.array(samples)
    return {"source": path.replace("/sys/class/drm/", ""), "samples": int(a.size),
            "median_mhz": float(np.median(a)), "p10_mhz": float(np.percentile(a, 10)),
            "p90_mhz": float(np.percentile(a, 90)), "nominal_mhz": NOMINAL_SCLK_MHZ,
            "what": "shader clock during back-to-back forwards of the headline workload"}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_single_thread():
    """Child process (OMP_NUM_THREADS=1, no GPU): the oracle on one thread, on
    the tiny layer (64 tokens, whole) and the dense linear (the first 128 rows
    of X [4096, 2048] against all of W [1536, 2048]).  Prints one JSON line."""
    import oracle
    import moe_workloads as W
    tw = W.tiny(seed=0)
    w1, w2 = tw.weights(threads=1)
    wts = oracle.DequantWeights(w1, w2)
    t0 = time.perf_counter()
    oracle.moe_forward(tw.x, tw.ids, tw.probs, wts)
    t_tiny = time.perf_counter() - t0
    dw = W.dense(seed=1)
    rows = 128
    xq, wq = oracle.quantize(dw.x[:rows]), oracle.quantize(dw.w)
    t0 = time.perf_counter()
    oracle.linear(xq, wq)
    t_dense = time.perf_counter() - t0
    print(json.dumps({"tiny_layer_tokens_per_s": tw.shape.T / t_tiny, "tiny_layer_s": t_tiny,
                      "dense_linear_gflop_per_s": 2.0 * rows * dw.N * dw.K / t_dense / 1e9, "dense_linear_s": t_dense,
                      "dense_sample": f"first {rows} of {dw.M} rows of X x all {dw.N} rows of W"}))


def cpu_baseline(wl, w1, w2, target_s):
    import oracle
    T = wl.shape.T
    wts = oracle.DequantWeights(w1, w2)  # weight quantization is outside the forward, as on the GPU

    def run(n):
        t0 = time.perf_counter()
        oracle.moe_forward(wl.x[:n], wl.ids[:n], wl.probs[:n], wts)
        return time.perf_counter() - t0

    n0 = 16
    t_small = run(n0)
    n = int(min(T, max(n0, n0 * target_s / max(t_small, 1e-3))))
    t = run(n) if n != n0 else t_small
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count()
    single = None
    try:
        import subprocess
        env = dict(os.environ, OMP_NUM_THREADS="1")
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--oracle-single-thread"], env=env,
                           capture_output=True, text=True, timeout=300)
        if r.returncode == 0:
            single = json.loads(r.stdout.strip().splitlines()[-1])
    except (OSError, ValueError, subprocess.SubprocessError):
        single = None
    return {"value": n / t, "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"first {n} of {T} tokens of the same workload (all their top-{wl.shape.K} pairs), "
                      f"weights pre-quantized and dequantized outside the timed region; {t:.1f} s",
            "single_thread": single}


def main():
    args = parse()
    if args.oracle_single_thread:
        oracle_single_thread()
        return
    if args.gpus != 1:
        print(f"bench.py: the expert forward runs on one GPU; --gpus {args.gpus} is not supported "
              "(expert-parallel sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    import torch

    import moe_workloads as W
    import nvfp4_moe_expert_sort_amd as m

    dev = torch.device("cuda:0")
    wl = W.qwen3(seed=2, T=args.tokens)
    s = wl.shape
    T, H, E, K, I = s.T, s.H, s.E, s.K, s.I
    w1, w2 = wl.weights(threads=16)
    cfg = m.make_config(H, I, E, K, T)
    w1_dev = torch.from_numpy(w1.view(np.int16)).to(dev)
    w2_dev = torch.from_numpy(w2.view(np.int16)).to(dev)
    qw = m.QuantWeights(cfg, dev).quantize_from(w1_dev, w2_dev)
    ws = m.alloc_workspace(cfg, dev)
    x = torch.from_numpy(wl.x.view(np.int16)).to(dev)
    ids = torch.from_numpy(wl.ids).to(dev)
    probs = torch.from_numpy(wl.probs).to(dev)
    out = torch.empty((T, H), dtype=torch.int16, device=dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    if args.calibrate_copy:
        src = torch.ones((1 << 30,), dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    # Weight quantization (once per weight update, outside the forward): W1 and W2
    # re-quantized in place, timed with events on the stream.
    wq = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    n_wq = 5
    wq[0].record(stream)
    for _ in range(n_wq):
        qw.quantize_from(w1_dev, w2_dev, stream=stream)
    wq[1].record(stream)
    torch.cuda.synchronize()
    wq_ms = wq[0].elapsed_time(wq[1]) / n_wq
    wq_rows = E * (2 * I + H)
    wq_bytes = 2 * E * (2 * I * H + H * I) + E * (2 * I * (H // 2 + H // 16) + H * (I // 2 + I // 16)) + 4 * wq_rows
    del w1_dev, w2_dev

    # The on-device router (secondary): FP32 scores of x against a [E, H] BF16
    # router weight (N(0, 0.02^2), seed 21) and the deterministic top-k with
    # renormalised probabilities, for the whole batch and at decode sizes.
    router = None
    if not args.no_router:
        rng = np.random.default_rng(21)
        w_r = torch.from_numpy(W.f32_to_bf16_bits((rng.standard_normal((E, H)) * 0.02).astype(np.float32))
                               .view(np.int16)).to(dev)
        router = {}
        for n in (T, 64, 1):
            xs = x[:n].contiguous()
            bufs = (torch.empty((n, E), dtype=torch.float32, device=dev),
                    torch.empty((n, K), dtype=torch.int32, device=dev),
                    torch.empty((n, K), dtype=torch.float32, device=dev))
            for _ in range(20):
                m.router_topk(xs, w_r, K, out=bufs)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(100):
                m.router_topk(xs, w_r, K, stream=stream, out=bufs)
            ev[1].record(stream)
            torch.cuda.synchronize()
            r_us = ev[0].elapsed_time(ev[1]) / 100 * 1e3
            r_bytes = n * H * 2 + E * H * 2 + n * E * 4 + n * K * 8
            router[f"T{n}"] = {"us": r_us, "tflops": 2.0 * n * H * E / (r_us / 1e6) / 1e12,
                               "GB_s": r_bytes / (r_us / 1e6) / 1e9,
                               "frac_hbm_peak": r_bytes / (r_us / 1e6) / 1e9 / HBM_PEAK_GBS}
        del w_r

    # Decode-sized forwards (secondary): the first n tokens of the workload, one
    # forward captured into a HIP graph and replayed back to back, and the same
    # forward launched eagerly; microseconds per forward.
    decode = {}
    if not args.no_decode:
        for n in (1, 8, 64):
            xs, ids_s, pr_s = x[:n].contiguous(), ids[:n].contiguous(), probs[:n].contiguous()
            out_s = torch.empty((n, H), dtype=torch.int16, device=dev)
            for _ in range(20):
                m.moe_expert_forward(cfg, xs, ids_s, pr_s, qw, ws, out=out_s)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            ev[0].record(stream)
            for _ in range(200):
                m.moe_expert_forward(cfg, xs, ids_s, pr_s, qw, ws, out=out_s, stream=stream)
            ev[1].record(stream)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                m.moe_expert_forward(cfg, xs, ids_s, pr_s, qw, ws, out=out_s)
            for _ in range(20):
                g.replay()
            ev[2].record(stream)
            for _ in range(200):
                g.replay()
            ev[3].record(stream)
            torch.cuda.synchronize()
            decode[f"T{n}"] = {"eager_us": ev[0].elapsed_time(ev[1]) / 200 * 1e3,
                               "graph_us": ev[2].elapsed_time(ev[3]) / 200 * 1e3}
            del g

    # Cold-cache forwards (secondary): a 512 MiB write evicts L2 and the 256 MB MALL before each one.
    cold = []
    if args.cold_steps > 0:
        scratch = torch.empty((512 << 20,), dtype=torch.uint8, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(5):
            m.moe_expert_forward(cfg, x, ids, probs, qw, ws, out=out)
        for _ in range(args.cold_steps):
            scratch.fill_(1)
            e0.record(stream)
            m.moe_expert_forward(cfg, x, ids, probs, qw, ws, out=out)
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        del scratch

    # The dense NVFP4 linear (secondary): X [4096, 2048] with 1 % outliers x50,
    # W [1536, 2048]; activation quantizer + one GEMM per call.
    dense = None
    if not args.no_dense:
        dw = W.dense(seed=1)
        xd = torch.from_numpy(dw.x.view(np.int16)).to(dev)
        wc, wsc, wg = m.quantize(torch.from_numpy(dw.w.view(np.int16)).to(dev), layout=m.LAYOUT_GEMM)
        Wq = m.qtensor(wc, wsc, wg, 1, dw.N, dw.K)
        lws = torch.empty((m.linear_workspace_bytes(dw.M, dw.K),), dtype=torch.uint8, device=dev)
        dout = torch.empty((dw.M, dw.N), dtype=torch.int16, device=dev)
        for _ in range(20):
            m.linear(xd, Wq, lws, out=dout)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(100):
            m.linear(xd, Wq, lws, out=dout, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        d_ms = ev[0].elapsed_time(ev[1]) / 100
        d_flop = 2.0 * dw.M * dw.N * dw.K
        dense = {"workload": dw.name, "ms": d_ms, "tflops": d_flop / (d_ms / 1e3) / 1e12,
                 "frac_f16_mfma_peak": d_flop / (d_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                 "what": "activation quantizer + one NVFP4 GEMM (f16 MFMA) per call"}
        del xd, wc, wsc, wg, lws, dout

    # Skewed routing (secondary): 16384 tokens whose expert popularity follows
    # Zipf(1.1) (some experts get 0-8 tokens, the hottest over 2000), on the same
    # quantized weights; tokens/s of the W4A4 forward.
    skewed = None
    if not args.no_skewed:
        sk = W.skewed(seed=3)
        ss = sk.shape
        cfg_s = m.make_config(H, I, E, K, ss.T)
        ws_s = m.alloc_workspace(cfg_s, dev)
        xs_ = torch.from_numpy(sk.x.view(np.int16)).to(dev)
        ids_ = torch.from_numpy(sk.ids).to(dev)
        pr_ = torch.from_numpy(sk.probs).to(dev)
        out_ = torch.empty((ss.T, H), dtype=torch.int16, device=dev)
        for _ in range(10):
            m.moe_expert_forward(cfg_s, xs_, ids_, pr_, qw, ws_s, out=out_)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(30):
            m.moe_expert_forward(cfg_s, xs_, ids_, pr_, qw, ws_s, out=out_, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        sk_ms = ev[0].elapsed_time(ev[1]) / 30
        cnt = sk.expert_counts()
        sk_tf = 2.0 * ss.T * K * 3 * H * I / (sk_ms / 1e3) / 1e12
        sk_bytes = layer_bytes(ss.T, H, E, K, I, cnt)["total"]
        skewed = {"workload": sk.name, "tokens": ss.T, "ms_per_step": sk_ms, "tokens_per_s": ss.T / (sk_ms / 1e3),
                  "tflops": sk_tf, "frac_f16_mfma_peak": sk_tf / MFMA_F16_PEAK_TFLOPS,
                  "frac_fp4_mfma_peak": sk_tf / MFMA_FP4_PEAK_TFLOPS,
                  "frac_hbm_peak": sk_bytes / (sk_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                  "expert_rows_min_max": [int(cnt.min()), int(cnt.max())]}
        del ws_s, xs_, ids_, pr_, out_

    # The W4A16 variant (secondary): the same workload with BF16 activations.
    w16 = None
    if not args.no_w4a16:
        for _ in range(20):
            m.moe_expert_forward_w4a16(cfg, x, ids, probs, qw, ws, out=out)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(50):
            m.moe_expert_forward_w4a16(cfg, x, ids, probs, qw, ws, out=out, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        w16_ms = ev[0].elapsed_time(ev[1]) / 50
        w16 = {"ms_per_step": w16_ms, "tokens_per_s": T / (w16_ms / 1e3),
               "tflops": 2.0 * T * K * 3 * H * I / (w16_ms / 1e3) / 1e12,
               "what": "NVFP4 weights x BF16 activations (bf16 MFMA), same routing, producer and combine"}

    # The forward with X's max, quantization and FC1 fused (secondary): the
    # same workload and output bits, X quantized inside FC1 instead of by the
    # sort and the gather.
    online = None
    if not args.no_online:
        for _ in range(20):
            m.moe_expert_forward_online(cfg, x, ids, probs, qw, ws, out=out)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(50):
            m.moe_expert_forward_online(cfg, x, ids, probs, qw, ws, out=out, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        on_ms = ev[0].elapsed_time(ev[1]) / 50
        online = {"ms_per_step": on_ms, "tokens_per_s": T / (on_ms / 1e3),
                  "what": "X's max in the sort, its quantization inside FC1 (no quantized copy of X, no gather); "
                          "outputs bitwise those of the headline forward"}

    # The BF16 straight-through backward (secondary): after the unfused forward
    # that stores y1, the backward of the same layer with a random upstream
    # gradient; dh, each pair's FC1 input gradient and both weight gradients
    # are 2 * T*K * 6 * H * I flop in BF16 MFMA.
    backward = None
    if not args.no_backward:
        w1_b = torch.from_numpy(w1.view(np.int16)).to(dev)
        w2_b = torch.from_numpy(w2.view(np.int16)).to(dev)
        out_u, y1_u = m.moe_expert_forward_unfused(cfg, x, ids, probs, qw, ws)
        rng = np.random.default_rng(32)
        dout = torch.from_numpy(W.f32_to_bf16_bits((rng.standard_normal((T, H)) * 0.1).astype(np.float32))
                                .view(np.int16)).to(dev)
        for _ in range(3):
            m.moe_expert_backward(cfg, x, w1_b, w2_b, y1_u, ws, dout)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        n_b = 10
        ev[0].record(stream)
        for _ in range(n_b):
            m.moe_expert_backward(cfg, x, w1_b, w2_b, y1_u, ws, dout, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        b_ms = ev[0].elapsed_time(ev[1]) / n_b
        b_flop = 2.0 * T * K * 6 * H * I
        backward = {"ms": b_ms, "tflops": b_flop / (b_ms / 1e3) / 1e12,
                    "frac_bf16_mfma_peak": b_flop / (b_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                    "what": "dx, router-probability and FP32 weight gradients; each call allocates its "
                            "outputs and workspace through torch (included)"}
        del w1_b, w2_b, out_u, y1_u, dout

    # The masked fixed-capacity layout (secondary): the same forward with expert
    # e's rows in the fixed chunk [e*capacity, (e+1)*capacity), capacity the
    # smallest multiple of 32 that holds the workload's busiest expert.
    masked = None
    if not args.no_masked:
        cap = int(-(-int(wl.expert_counts().max()) // 32) * 32)
        ws_m = m.alloc_workspace_masked(cfg, cap, dev)
        for _ in range(20):
            m.moe_expert_forward_masked(cfg, cap, x, ids, probs, qw, ws_m, out=out)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for _ in range(50):
            m.moe_expert_forward_masked(cfg, cap, x, ids, probs, qw, ws_m, out=out, stream=stream)
        ev[1].record(stream)
        torch.cuda.synchronize()
        mk_ms = ev[0].elapsed_time(ev[1]) / 50
        masked = {"capacity": cap, "ms_per_step": mk_ms, "tokens_per_s": T / (mk_ms / 1e3),
                  "what": "same workload, expert rows in fixed chunks of `capacity` (static-capacity layout)"}
        del ws_m

    # Order: the light secondaries (router, decode sizes) first, the full-size
    # ones after, the masked forward last, so the GPU enters the headline's
    # warm-up and timed forwards at the clock it holds under sustained load.
    for _ in range(args.warmup):
        m.moe_expert_forward(cfg, x, ids, probs, qw, ws, out=out)
    torch.cuda.synchronize()
    if m.device_error(cfg, ws) != 0:
        raise RuntimeError("device error word set")

    # Timed region: exactly `steps` plain forwards, bracketed by device syncs.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        m.moe_expert_forward(cfg, x, ids, probs, qw, ws, out=out, stream=stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Stage breakdown in a separate pass (not part of `value`): the same forward
    # with HIP events recorded on its stream at the stage boundaries.  Each
    # event adds a few microseconds between kernels, so these forwards are a
    # little slower than the timed ones; the kernels' own durations are not.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(m.N_STAGE_EVENTS)] for _ in range(args.steps)]
    for ev in events:  # torch creates the underlying hipEvent on first record
        for e in ev:
            e.record(stream)
    torch.cuda.synchronize()
    for k in range(args.steps):
        m.moe_expert_forward_events(cfg, x, ids, probs, qw, ws, events[k], out, stream=stream)
    torch.cuda.synchronize()
    stage_ms = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(m.N_STAGE_EVENTS - 1)] for ev in events])
    stage_mean = stage_ms.mean(axis=0)

    def _fwd_batch():
        for _ in range(10):
            m.moe_expert_forward(cfg, x, ids, probs, qw, ws, out=out, stream=stream)
        torch.cuda.synchronize()
    clock = observed_clock(_fwd_batch)

    P = T * K
    layer_flop = 2.0 * P * 3 * H * I
    fc1_flop = 2.0 * P * H * 2 * I
    fc2_flop = 2.0 * P * I * H
    fc1_s = stage_mean[1] / 1e3
    achieved = fc1_flop / fc1_s / 1e12
    counts = wl.expert_counts()
    byts = layer_bytes(T, H, E, K, I, counts)
    layer_s = ms_per_step / 1e3
    result = {
        "metric": "NVFP4 MoE expert-forward tokens/s (FC1+FC2) and % of MFMA peak",
        "value": T / layer_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4(e2m1 x e4m3) -> f16 mfma, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) random weights, softmax top-8 routing)",
        "config": {"workload": wl.name, "tokens": T, "hidden": H, "experts": E, "top_k": K, "inter": I,
                   "seed": 2, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": fc1_traffic_bytes(),
                     "traffic_unit": "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_bytes": byts["fc1"],
                     "kernel": "gemm_kernel<SwiGLU> (FC1 grouped GEMM + router-weighted SwiGLU producer)",
                     "work_per_launch": f"2*T*K*H*2I = {fc1_flop:.4e} flop (useful rows only)",
                     "avg_launch_ms": stage_mean[1],
                     "frac_at_observed_clock": (achieved / (MFMA_F16_PEAK_TFLOPS * clock["median_mhz"] / NOMINAL_SCLK_MHZ)
                                                if clock else None)},
        "clock": clock,
        "layer": {"tflops": layer_flop / layer_s / 1e12,
                  "frac_f16_mfma_peak": layer_flop / layer_s / 1e12 / MFMA_F16_PEAK_TFLOPS,
                  "frac_fp4_mfma_peak": layer_flop / layer_s / 1e12 / MFMA_FP4_PEAK_TFLOPS,
                  "hbm_gbs_algorithmic": byts["total"] / layer_s / 1e9,
                  "frac_hbm_peak": byts["total"] / layer_s / 1e9 / HBM_PEAK_GBS,
                  "stage_ms": dict(zip(m.STAGES, [round(float(v), 4) for v in stage_mean])),
                  "fc2_tflops": fc2_flop / (stage_mean[3] / 1e3) / 1e12,
                  "cold_ms_median": float(np.median(cold)) if cold else None,
                  "cold_ms_p10_p90": [float(np.percentile(cold, 10)), float(np.percentile(cold, 90))] if cold else None,
                  "cold_forwards": len(cold),
                  "cold_tokens_per_s": T / (np.median(cold) / 1e3) if cold else None},
        "weight_quantization": {"ms": wq_ms, "bytes": wq_bytes, "GB_s": wq_bytes / (wq_ms / 1e3) / 1e9,
                                "frac_hbm_peak": wq_bytes / (wq_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                "what": "W1 [E,2I,H] and W2 [E,H,I] BF16 read, NVFP4 codes/scales/g written"},
    }
    if decode:
        result["decode"] = decode
    if masked:
        result["masked"] = masked
    if router:
        result["router"] = router
    if backward:
        result["backward"] = backward
    if w16:
        result["w4a16"] = w16
    if online:
        result["online_fc1_quant"] = online
    if dense:
        result["dense_linear"] = dense
    if skewed:
        result["skewed"] = skewed
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, w1, w2, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
