"""The owner step under HIP graph capture.

With its descriptors already resident in the workspace and no phase events
requested, mfsdp_owner_step enqueues nothing but kernel launches on the
caller's stream (no copies, no memsets, no allocation), so a caller can
capture it into a graph and replay it.  Launch arguments are fixed at
capture: the same buffers, and for an AdamW tail the same bias-correction
step, so the table here has Muon matrices only.
"""

import pytest

from matrix_optimizer_owner_amd import binding as B
from matrix_optimizer_owner_amd import workloads as W
from tests.harness import DeviceRun, say

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager_bitwise():
    """Eager and graph-replayed trajectories over four steps of fresh
    gradients are bitwise equal after every step; between replays the
    program does its own eager work (the gradient refill) and synchronises."""
    specs = [s for s in W.config(1).specs if s.rows > 1 and s.cols > 1]
    wl = W.Workload("gpt2-matrices", specs, seed=1, hparams=dict(W.MUON_DEFAULTS, ns_precision=0))
    a, b = DeviceRun(wl), DeviceRun(wl)
    torch = a.torch
    try:
        for r in (a, b):
            r.fill(1, params_too=True)
            r.run(1)  # uploads the descriptors
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            b.run(2, flags=B.STEP_DESCRIPTORS_RESIDENT)
        torch.cuda.synchronize()
        for t in range(2, 6):
            a.fill(t, params_too=False)
            a.run(t, flags=B.STEP_DESCRIPTORS_RESIDENT)
            b.fill(t, params_too=False)
            graph.replay()
            torch.cuda.synchronize()
            for name in ("params", "state", "ns_out"):
                x, y = getattr(a, name), getattr(b, name)
                same = bool(torch.equal(x.view(torch.uint8), y.view(torch.uint8)))
                say(f"  step {t} {name}: graph replay bitwise equal to eager = {same}")
                assert same, (t, name)
        graph.reset()
    finally:
        a.free()
        b.free()
