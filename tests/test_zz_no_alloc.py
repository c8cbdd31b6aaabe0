"""The step that allocates nothing (mfsdp_owner_step_static, the library's
own workspace) against mfsdp_owner_step (a caller workspace) on the same
inputs, through the C ABI: two calls in a row, the second with a smaller
table, each bitwise equal to the caller-workspace step (same kernels, and the
step is deterministic), and each checked against the fp64 oracle as every
other step is; then the first table again with the resident-descriptor flag
after the other plan has used the array (the library must upload again);
and a plan larger than the static workspace, or a workspace pointer passed
to the static call, refused before any GPU work."""

import numpy as np
import pytest

from matrix_optimizer_owner_amd import binding as B
from matrix_optimizer_owner_amd import workloads as W
from tests.harness import DeviceRun, assert_reports, check_step, say
from tests.test_random_shapes_gpu import random_table

pytestmark = pytest.mark.gpu


def _step(run, t, static, flags=0):
    import torch

    stream = torch.cuda.current_stream().cuda_stream
    if static:
        run.plan.step_static(run.params.data_ptr(), run.grads.data_ptr(), run.state.data_ptr(), t, stream=stream,
                             ns_out=run.ns_out.data_ptr(), flags=flags)
    else:
        run.run(t)


def _pair(wl, label):
    """A fresh run of each entry point from the same inputs; returns both."""
    runs = {}
    for static in (False, True):
        run = DeviceRun(wl)
        assert run.plan.workspace_bytes <= B.STATIC_WORKSPACE_BYTES
        run.fill(1, params_too=True)
        before = run.host()
        _step(run, 1, static)
        after = run.host()
        assert_reports(check_step(run, before, after, 1), f"{label} static={static}")
        runs[static] = (run, after)
    return runs


def _same(a, b, label):
    for k in ("params", "state", "ns_out"):
        x, y = np.ascontiguousarray(a[k]).view(np.uint8), np.ascontiguousarray(b[k]).view(np.uint8)
        same = x.shape == y.shape and bool(np.array_equal(x, y))
        say(f"  [{label}] {k}: bitwise equal = {same}")
        assert same, f"{label}: {k} differs"


def test_static_workspace_step_matches_caller_workspace_step():
    big, small = random_table(21, 0), W.small_ragged(precision=0)
    say(f"[no-alloc] first call: {big.name}; second call: {small.name}")
    r1 = _pair(big, "first (larger)")
    _same(r1[False][1], r1[True][1], "first (larger)")
    r2 = _pair(small, "second (smaller)")
    _same(r2[False][1], r2[True][1], "second (smaller)")
    # the larger table once more, flagged resident: the array now holds the
    # smaller plan's descriptors, so the library uploads this plan's again
    for static in (False, True):
        run, _ = r1[static]
        run.fill(2, params_too=False)
        _step(run, 2, static, flags=B.STEP_DESCRIPTORS_RESIDENT)
    _same(r1[False][0].host(), r1[True][0].host(), "larger again, resident flag")
    for r in (r1, r2):
        for run, _ in r.values():
            run.free()


def test_static_workspace_refusals():
    wl = W.config(1)  # GPT-2-small owner buffer: 432 MiB of workspace
    run = DeviceRun(wl)
    try:
        assert run.plan.workspace_bytes > B.STATIC_WORKSPACE_BYTES
        run.fill(1, params_too=True)
        with pytest.raises(B.MfsdpError) as ei:
            _step(run, 1, True)
        assert ei.value.status == 5 and "static workspace" in ei.value.message
        small = DeviceRun(W.small_ragged(precision=0))
        args = B.StepArgs(small.params.data_ptr(), small.grads.data_ptr(), small.state.data_ptr(),
                          small.ws.data_ptr(), small.ws_bytes, 1, None, None, 0, None, 0)
        import ctypes

        st = B.load().mfsdp_owner_step_static(small.plan._h, ctypes.byref(args))
        assert st == 1
        small.free()
    finally:
        run.free()
