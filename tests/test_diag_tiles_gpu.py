"""GPU parity where diagonal tiles carry the Gram and the polynomial.

On a diagonal tile (row block = column block) both operands of C = P Q^T are
the same rows of the same matrix, and the kernels then stage only P and read
both fragments from it.  These tables are made of matrices whose Gram and
polynomial are one diagonal tile (or two diagonal tiles and one off the
diagonal) with contractions long enough to run many stages through that
path, on each tile edge, against the fp64 oracle, two teacher-forced steps.
"""

import pytest

from matrix_optimizer_owner_amd import workloads as W
from tests.harness import DeviceRun, assert_reports, check_step, say

pytestmark = pytest.mark.gpu


def diag_table(precision: int) -> W.Workload:
    sp = [
        W.TensorSpec("w_256x4096", 256, 4096, grad_std=1e-3),      # one 256 Gram tile, 64 stages
        W.TensorSpec("w_3000x200", 3000, 200, grad_std=1e-2),      # tall, padded to 256 x 3072
        W.TensorSpec("w_128x2048", 128, 2048, "f32", grad_std=1e-3),
        W.TensorSpec("w_97x1500", 97, 1500, grad_std=1e-1),
        W.TensorSpec("b_777", 1, 777, "f32", grad_std=1e-3),
    ]
    return W.Workload(f"diag-tiles-p{precision}", sp, seed=31, hparams=dict(W.MUON_DEFAULTS, ns_precision=precision))


@pytest.mark.parametrize("tile", ["256", "128"])
def test_diagonal_tiles_bf16(tile):
    wl = diag_table(0)
    run = DeviceRun(wl, {"ns_tile": int(tile)})
    for t in (1, 2):
        say(f"[diag-tiles tile={tile}] step {t}: {wl.name}")
        run.fill(t, params_too=(t == 1))
        before = run.host()
        run.run(t)
        after = run.host()
        assert_reports(check_step(run, before, after, t), f"diag-tiles tile={tile} t={t}")
