"""Calls captured into a HIP graph (as bench.py times them, and as callers that cannot allocate run
them) give the eager result on every replay.

Each graph is replayed several times, with the program's own eager work (other library calls on
other buffers, torch ops) and synchronisations between the replays; every replay's output must equal
the eager output bit for bit (same kernels, same inputs).
"""
import pytest
import torch

import sliding_window_attention_index_amd as sattn
import workloads as W
from parity import SINK_NAMES

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    sattn.load_library()
    return torch.device("cuda:0")


def _replays_equal(dev, run, out, eager, noise):
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        run()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(float("nan") if out.is_floating_point() else -7)
        noise(r)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {r} differs from the eager call"


def _noise_window(dev):
    c = W.make_window_case("noise", [300, 77], 16, 8, 128, 128, 128, W.SINK_KEY0, seed=31)
    q, k, v, cu, s = (t.to(dev) for t in (c.q, c.k, c.v, c.cu_seqlens, c.sinks))

    def noise(r):
        sattn.window_fwd(q, k, v, cu, c.max_seqlen, window=(128, 128), sinks=s, sink_mode="key0")
        (q.float() * (r + 1)).sum()
    return noise


def test_graph_window(dev):
    c = W.make_window_case("graph_win", [1500, 700, 64], 16, 8, 128, 128, 128, W.SINK_KEY0, seed=30)
    q, k, v, cu, s = (t.to(dev) for t in (c.q, c.k, c.v, c.cu_seqlens, c.sinks))
    out = torch.empty_like(q)

    def run():
        sattn.window_fwd(q, k, v, cu, c.max_seqlen, window=(128, 128), sinks=s, sink_mode="key0", out=out)
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    _replays_equal(dev, run, out, eager, _noise_window(dev))


@pytest.mark.parametrize("mode", [W.SINK_NONE, W.SINK_NULL])
@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_indexed_split(dev, mode, noalloc):
    """The decode shape (8 slices + merge), through the workspace call and the no-allocation call."""
    c = W.sparse_decode_case(seed=5, sink_mode=mode, name="graph_decode")
    q, kv, idx = c.q.to(dev), c.kv.to(dev), c.topk_idxs.to(dev)
    sinks = c.sinks.to(dev) if c.sinks is not None else None
    B, M, H, D, N, K = c.dims
    out = torch.empty_like(q)
    ws = torch.empty(sattn.indexed_workspace_size(B, M, H, D, 8), dtype=torch.uint8, device=dev)

    def run():
        if noalloc:
            sattn.indexed_fwd_noalloc(q, kv, idx, out=out, sinks=sinks, sink_mode=SINK_NAMES[mode], num_splits=8)
        else:
            sattn.indexed_fwd(q, kv, idx, sinks=sinks, sink_mode=SINK_NAMES[mode], num_splits=8, out=out,
                              workspace=ws)
    run()
    torch.cuda.synchronize()
    eager = out.clone()
    other = W.sparse_decode_case(seed=6, batch=8, name="noise")
    oq, okv, oidx = other.q.to(dev), other.kv.to(dev), other.topk_idxs.to(dev)

    def noise(r):
        sattn.indexed_fwd(oq, okv, oidx, num_splits=3 + r)
        torch.randn(1 << 20, device=dev).sum()
    _replays_equal(dev, run, out, eager, noise)
