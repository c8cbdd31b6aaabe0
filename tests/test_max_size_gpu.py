"""GPU parity at the largest matrix the planner accepts.

The planner rejects a Muon matrix whose padded Newton-Schulz buffer (bf16,
both dimensions rounded up to 256) reaches 2 GiB, because the contraction
kernels address one operand matrix with 32-bit byte offsets and the final
update indexes W with 32-bit element offsets.  These cases sit just under
that limit with ragged dimensions (neither a multiple of 256), wide and tall,
so the edge tiles, the transposed parameter write and the largest offsets
all run: padded 32512 x 32768, 2,130,706,432 bytes per X^T buffer.

Two Newton-Schulz iterations (the oracle's vector-applied iteration finishes
them on a 1.06 G-element matrix in about a minute): O V for four random
vectors against the oracle, plus sampled momentum and parameter elements.
"""

import numpy as np
import pytest

from matrix_optimizer_owner_amd import workloads as W
from oracle import muon_oracle as orc
from tests.harness import DeviceRun, oracle_hparams, say
from tests.test_parity_full_gpu import check_elementwise, normalised_input

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.mark.parametrize("rows,cols", [(32500, 32700), (32700, 32500)])
def test_largest_accepted_matrix(rows, cols):
    wl = W.Workload(f"max-{rows}x{cols}", [W.TensorSpec("w", rows, cols, grad_std=1e-4)], seed=6,
                    hparams=dict(W.MUON_DEFAULTS, ns_precision=0))
    run = DeviceRun(wl, {"ns_steps": 2})
    hp = oracle_hparams(run.hp)
    say(f"[max-size] {rows}x{cols} bf16, workspace {run.ws_bytes / 2**30:.2f} GiB")
    rng = np.random.default_rng(rows)
    try:
        run.fill(1, params_too=True)
        snap = run.snapshot_entries([0])
        run.run(1)
        o = check_elementwise(run, snap, 0, hp, rng)
        x0 = normalised_input(snap, 0, hp)
        del snap
        v = rng.standard_normal((cols, 4))
        want = orc.newton_schulz_apply(x0, v, 2, hp.ns_a, hp.ns_b, hp.ns_c)
        rel = np.linalg.norm(o @ v - want) / np.linalg.norm(want)
        say(f"  |O V - NS2(X) V| / |NS2(X) V| = {rel:.3e}")
        assert rel <= 3e-2
    finally:
        run.free()
