"""GPU parity on seeded random owner tables: many ragged shapes at once.

Each table mixes seeded random Muon matrices (each dimension 2-1200, tall,
wide and square, none a multiple of the tile on purpose except by chance),
fixed extremes (2 x 2, 2 x 1199, 1199 x 2, 255 x 257, 257 x 255, 1 x 1),
fp32 and bf16 parameters and AdamW vectors, packed at random 16-byte-aligned
gaps.  Two teacher-forced steps through the whole oracle, on the planner's
own tile choice and with the 256-tile kernels forced.
"""

import numpy as np
import pytest

from matrix_optimizer_owner_amd import workloads as W
from tests.harness import DeviceRun, assert_reports, check_step, say

pytestmark = pytest.mark.gpu


class _Packed(W.Workload):
    """A workload whose entries sit at given offsets (gaps between them)."""

    def __init__(self, name, specs, seed, hparams, gaps):
        super().__init__(name, specs, seed, hparams=hparams)
        self.gaps = gaps

    def layout(self):
        offs, off = [], 0
        for s, g in zip(self.specs, self.gaps):
            off += g
            offs.append(off)
            off = (off + s.numel * s.itemsize + 15) // 16 * 16
        return offs, max(off, 256)


def random_table(seed: int, precision: int) -> W.Workload:
    rng = np.random.default_rng(seed)
    sp = []
    for k in range(14):
        r, c = (int(x) for x in rng.integers(2, 1201, 2))
        dt = "f32" if rng.random() < 0.25 else "bf16"
        sp.append(W.TensorSpec(f"rand{k}_{r}x{c}", r, c, dt, grad_std=float(10.0 ** rng.uniform(-4, 0))))
    for r, c in ((2, 2), (2, 1199), (1199, 2), (255, 257), (257, 255)):
        sp.append(W.TensorSpec(f"edge_{r}x{c}", r, c, grad_std=1e-3))
    sp += [W.TensorSpec("scalar", 1, 1, "f32", grad_std=1e-3), W.TensorSpec("vec_bf16", 1, 777, "bf16", grad_std=1e-3),
           W.TensorSpec("vec_f32", 333, 1, "f32", "ones", grad_std=1e-3)]
    order = rng.permutation(len(sp))
    sp = [sp[i] for i in order]
    gaps = [int(g) * 16 for g in rng.integers(0, 4, len(sp))]
    return _Packed(f"random-table-s{seed}-p{precision}", sp, seed, dict(W.MUON_DEFAULTS, ns_precision=precision), gaps)


@pytest.mark.parametrize("seed,precision,tile", [(21, 0, None), (22, 0, "256"), (23, 1, None), (24, 0, "256"),
                                                 (25, 0, "256"), (26, 1, "256"), (27, 0, "128")])
def test_random_tables(seed, precision, tile):
    wl = random_table(seed, precision)
    run = DeviceRun(wl, {"ns_tile": int(tile)} if tile else None)
    try:
        for t in (1, 2):
            say(f"[random s{seed} p{precision} tile={tile}] step {t}: {[(s.rows, s.cols) for s in wl.specs]}")
            run.fill(t, params_too=(t == 1))
            before = run.host()
            run.run(t)
            after = run.host()
            assert_reports(check_step(run, before, after, t), f"random s{seed} t={t}")
    finally:
        run.free()
