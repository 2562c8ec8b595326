"""The expert forward captured into a HIP graph and replayed.

The forward allocates nothing, reads nothing back to the host and issues no
memory fills (article section 4.6: expert boundaries stay device offsets and
capacities are static, which is what makes the decode path capturable), so a
graph captured once can be replayed with new inputs copied into its input
buffers.  Each replay must reproduce, bit for bit, an eager forward of the
same inputs with its own workspace; eager work and synchronisations run
between the replays."""
import numpy as np
import pytest

import moe_workloads as W
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import nvfp4_moe_expert_sort_amd as m
    m.lib()
    dev = torch.device("cuda:0")
    s = W.qwen3(seed=2, T=1).shape
    w1, w2 = W.qwen3(seed=2, T=1).weights(threads=16)
    cfg = m.make_config(s.H, s.I, s.E, s.K, 2048)
    qw = m.QuantWeights(cfg, dev).quantize_from(to_dev(w1, dev), to_dev(w2, dev))
    return m, dev, cfg, qw


@pytest.mark.parametrize("T", [1, 96, 2048])
def test_graph_replay_matches_eager(layer, T):
    import torch
    m, dev, cfg, qw = layer
    base = W.qwen3(seed=2, T=T)
    ws_graph = m.alloc_workspace(cfg, dev)
    ws_eager = m.alloc_workspace(cfg, dev)
    x = to_dev(base.x, dev)
    ids = to_dev(base.ids, dev)
    probs = to_dev(base.probs, dev)
    out = torch.empty((T, cfg.hidden), dtype=torch.int16, device=dev)

    # an eager call first loads the kernels; then capture on torch's side stream
    m.moe_expert_forward(cfg, x, ids, probs, qw, ws_graph, out=out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        m.moe_expert_forward(cfg, x, ids, probs, qw, ws_graph, out=out)
    torch.cuda.synchronize()

    prev = None
    for seed in (5, 6, 7):
        wl = W.qwen3(seed=seed, T=T)
        x.copy_(to_dev(wl.x, dev))
        ids.copy_(to_dev(wl.ids, dev))
        probs.copy_(to_dev(wl.probs, dev))
        graph.replay()
        torch.cuda.synchronize()
        ref = m.moe_expert_forward(cfg, to_dev(wl.x, dev), to_dev(wl.ids, dev), to_dev(wl.probs, dev), qw, ws_eager)
        torch.cuda.synchronize()
        assert m.device_error(cfg, ws_graph) == 0
        assert torch.equal(out, ref), f"replay with inputs of seed {seed} differs from the eager forward"
        # the replay recomputed: inputs of another seed give another output
        if prev is not None:
            assert not torch.equal(out, prev), "replay left the previous output in place"
        prev = out.clone()
    print(f"  T={T}: 3 graph replays == eager forward, bit for bit")


def test_concurrent_streams_with_separate_workspaces(layer):
    """Two forwards in flight at once on two streams, each with its own
    workspace (the library keeps no mutable global state): each equals the
    same forward run alone."""
    import torch
    m, dev, cfg, qw = layer
    wa, wb = W.qwen3(seed=8, T=2048), W.qwen3(seed=9, T=1500)
    ins = [(to_dev(w.x, dev), to_dev(w.ids, dev), to_dev(w.probs, dev)) for w in (wa, wb)]
    ws = [m.alloc_workspace(cfg, dev) for _ in range(2)]
    ref = []
    for (x, ids, probs), w in zip(ins, ws):
        ref.append(m.moe_expert_forward(cfg, x, ids, probs, qw, w))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(r) for r in ref]
    for rep in range(3):
        for (x, ids, probs), w, st, o in zip(ins, ws, streams, outs):
            with torch.cuda.stream(st):
                m.moe_expert_forward(cfg, x, ids, probs, qw, w, out=o, stream=st)
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"repetition {rep}"
