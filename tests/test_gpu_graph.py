"""The decode step is fixed-shape and sync-free (FreeToken PR #499, "Design":
fixed-shape kernels, graph-safe): it can be captured in a HIP graph, and
replays -- with eager work on the same stream between them -- give exactly
the eager results."""
import numpy as np
import pytest
import torch

from workload import get_workload

from tests.gpu_compare import say

pytestmark = pytest.mark.gpu

OUTS = ("sel", "needed", "out_slots", "miss_count", "out")


def _snapshot(g):
    return {k: getattr(g, k).clone() for k in OUTS}


def test_captured_steps_replay_like_eager():
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3s")
    say("[graph] capture c3s decode steps")
    eager, graphed = GpuWorkload(wl), GpuWorkload(wl)
    for g in (eager, graphed):
        g.setup()
        g.upload_queries()
    torch.cuda.synchronize()
    graphs = []
    for s in range(wl.steps):
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg):
            graphed.decode_step(s)
        graphs.append(cg)
    torch.cuda.synchronize()
    for s in range(wl.steps):
        eager.decode_step(s)
        graphs[s].replay()
        _ = graphed.tier.read_counters()          # eager work between replays
        torch.cuda.synchronize()
        a, b = _snapshot(eager), _snapshot(graphed)
        for k in OUTS:
            assert torch.equal(a[k], b[k]), f"step {s}: {k}"
    sa, sb = eager.tier.read_state(), graphed.tier.read_state()
    for k in ("page_to_slot", "slot_to_page", "stamp"):
        assert np.array_equal(sa[k], sb[k]), k
    assert eager.tier.read_counters() == graphed.tier.read_counters()


def test_one_graph_replayed_repeatedly():
    """The same captured step replayed three times == the same step run
    eagerly three times (the LRU state moves on each time)."""
    from workload.gpu_run import GpuWorkload
    wl = get_workload("c3s")
    say("[graph] repeated replay")
    eager, graphed = GpuWorkload(wl), GpuWorkload(wl)
    for g in (eager, graphed):
        g.setup()
        g.upload_queries()
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        graphed.decode_step(2)
    for _ in range(3):
        eager.decode_step(2)
        cg.replay()
        torch.cuda.synchronize()
        a, b = _snapshot(eager), _snapshot(graphed)
        for k in OUTS:
            assert torch.equal(a[k], b[k]), k
