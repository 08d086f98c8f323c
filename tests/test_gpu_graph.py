"""Steps captured as HIP graphs: every replay must give exactly what the same steps give
launched call by call.  Workload 2's step (MiniGPT layer set, delayed scaling, forward and
backward: 9 cast-transposes, 9 GEMMs, the recipe update) on one stream and forked over three,
workload 1's 16-step loop (per-tensor quantize of X and W, GEMM, update), and workload 3's
blockwise training step (3 blockwise cast-transposes, 3 GEMMs) on one stream and on three.

The steps are the ones bench.py times.  Their entry points allocate nothing and record no
memset, so every call goes into the graph.  The
replays run with eager device work and host synchronisation between them, and each replay's
recipe state (history, scales), codes and GEMM outputs are compared bit for bit with the
matching eager step from the same starting state."""

import pytest
import torch

pytestmark = pytest.mark.gpu

from gpu_util import DEV, announce  # noqa: E402


def _snapshot(step):
    return [t.detach().clone() for t in step.outputs()]


@pytest.mark.parametrize("streams", [1, 3])
def test_minigpt_step_graph_replays_match_eager(streams):
    """streams=3: each layer's casts and GEMMs forked over three streams and joined by events,
    so the graph holds a DAG; its replays must still equal the eager steps bit for bit."""
    import bench
    import scaled_quantize_gemm_amd as sq
    import workloads

    announce("graph: MiniGPT step, eager reference, streams", streams)
    step = bench.MiniGPTStep(sq, workloads, torch.device(DEV), streams=streams)
    st = step.state
    start = [st.amax_history.clone(), st.scale.clone(), st.scale_inv.clone()]
    n = 3
    eager = []
    for _ in range(n):
        step()
        torch.cuda.synchronize()
        eager.append(_snapshot(step))
    # the recipe state moved on every step, so the steps differ from one another
    assert not torch.equal(eager[0][1], eager[-1][1]) or not torch.equal(eager[0][0], eager[-1][0])

    announce("graph: capture, streams", streams)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    # capture launches nothing: back to the starting state, in place (the graph holds addresses)
    for dst, src in zip((st.amax_history, st.scale, st.scale_inv), start):
        dst.copy_(src)
    torch.cuda.synchronize()
    for k in range(n):
        announce("graph: replay", k, "streams", streams)
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(step)
        for i, (a, b) in enumerate(zip(got, eager[k])):
            assert a.dtype == b.dtype and a.shape == b.shape
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {k}: output {i} differs"
        # eager work of the program's own between replays
        torch.ones(1 << 20, device=DEV).mul_(2.0).sum().item()


def test_workload1_loop_graph_replays_match_eager():
    """Workload 1's 16 steps (per-tensor fp8_quantize of X and W, GEMM, recipe update) captured
    as one graph: two replays from the starting state equal eager steps 1-16 and 17-32."""
    import bench
    import scaled_quantize_gemm_amd as sq
    import workloads

    announce("graph: workload 1 loop, eager reference")
    step = bench.Workload1Step(sq, workloads, torch.device(DEV))
    st = step.state
    start = [st.amax_history.clone(), st.scale.clone(), st.scale_inv.clone()]
    eager = []
    for _ in range(2):
        for _ in range(16):
            step()
        torch.cuda.synchronize()
        eager.append(_snapshot(step))
    assert step.t == 0
    announce("graph: workload 1 capture")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(16):
            step()
    torch.cuda.synchronize()
    for dst, src in zip((st.amax_history, st.scale, st.scale_inv), start):
        dst.copy_(src)
    torch.cuda.synchronize()
    for k in range(2):
        announce("graph: workload 1 replay", k)
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_snapshot(step), eager[k])):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {k}: output {i} differs"
        torch.ones(1 << 20, device=DEV).mul_(2.0).sum().item()


@pytest.mark.parametrize("streams", [1, 3])
def test_blockwise_step_graph_replays_match_eager(streams):
    """Workload 3's blockwise training step (three blockwise cast-transposes feeding the forward,
    dgrad and wgrad GEMMs), on one stream and forked over three: two graph replays, with eager
    work between them, equal the eager step bit for bit (current scaling: no state between
    steps)."""
    import bench
    import scaled_quantize_gemm_amd as sq
    import workloads

    announce("graph: blockwise step, eager reference, streams", streams)
    step = bench.BlockwiseStep(sq, workloads, torch.device(DEV), streams=streams)
    step()
    torch.cuda.synchronize()
    eager = _snapshot(step)
    for t in step.outputs():  # the replays must rewrite every output
        t.zero_()
    announce("graph: blockwise capture, streams", streams)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for k in range(2):
        announce("graph: blockwise replay", k, "streams", streams)
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(_snapshot(step), eager)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {k}: output {i} differs"
        torch.ones(1 << 20, device=DEV).mul_(2.0).sum().item()
