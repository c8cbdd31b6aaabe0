"""GPU parity: the HIP owner step through the C ABI against the fp64 oracle,
teacher-forced, on seeded synthetic owner buffers."""

import numpy as np
import pytest

from matrix_optimizer_owner_amd import workloads as W
from tests.harness import DeviceRun, assert_reports, check_step, say

pytestmark = pytest.mark.gpu


def _run_steps(wl, steps, hp_overrides=None, label=""):
    run = DeviceRun(wl, hp_overrides)
    for t in range(1, steps + 1):
        say(f"[{label}] step {t}: {wl.name}")
        run.fill(t, params_too=(t == 1))
        before = run.host()
        run.run(t)
        after = run.host()
        assert_reports(check_step(run, before, after, t), f"{label} t={t}")
    return run


def test_small_ragged_bf16():
    _run_steps(W.small_ragged(precision=0), 2, label="ragged-bf16")


def test_small_ragged_fp32():
    _run_steps(W.small_ragged(precision=1), 2, label="ragged-fp32")


def test_single_fp32_config():
    _run_steps(W.config(0), 1, label="single-fp32")


def test_gpt2_small_owner_buffer():
    _run_steps(W.config(1), 1, label="gpt2")
