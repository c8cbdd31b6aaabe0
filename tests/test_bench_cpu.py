"""CPU checks of the benchmark's contract and of the workload accounting it
reports (no GPU needed).

* ``bench.py --gpus 2`` exits with status 2 and says why: the owner step has
  no cross-GPU work, and one GPU is what this build measures.
* The workloads' nominal Newton-Schulz FLOPs (5 iterations of 4 m^2 n + 2 m^3
  per matrix, m = min dim) and element counts match the figures the
  workload descriptions fix: GPT-2-small 48 matrices of 768 x {2304, 768,
  3072, 3072}; the Llama-3-8B share 4 layers of 4096^2 (q, o), 1024 x 4096
  (k, v), 14336 x 4096 (gate, up) and 4096 x 14336 (down); the Llama-3-70B
  share 2 layers of 8192^2, 1024 x 8192, 28672 x 8192 and 8192 x 28672.
  The expected values are written out here from those shapes, not taken
  from the code under test.
* The traffic record is keyed to the sources digest and is reported only
  while the digest matches.
"""

import os
import subprocess
import sys

import pytest

from matrix_optimizer_owner_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _ns(shapes, steps=5):
    return steps * sum(4.0 * min(r, c) ** 2 * max(r, c) + 2.0 * min(r, c) ** 3 for r, c in shapes)


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, cwd=ROOT, env=dict(os.environ, WORLD_SIZE="1"))
    assert res.returncode == 2
    assert "one GPU" in res.stderr


@pytest.mark.parametrize("cfg,shapes,elements", [
    (1, [(768, 2304), (768, 768), (768, 3072), (3072, 768)] * 12, 84_934_656),
    (2, ([(4096, 4096)] * 2 + [(1024, 4096)] * 2 + [(14336, 4096)] * 2 + [(4096, 14336)]) * 4, 872_415_232),
    (4, ([(8192, 8192)] * 2 + [(1024, 8192)] * 2 + [(28672, 8192)] * 2 + [(8192, 28672)]) * 2, 1_711_276_032),
])
def test_nominal_flops_and_elements(cfg, shapes, elements):
    wl = W.config(cfg)
    got = sorted((s.rows, s.cols) for s in wl.muon_specs())
    assert got == sorted(shapes)
    assert wl.muon_elements() == elements
    assert wl.nominal_ns_flops() == pytest.approx(_ns(shapes), rel=1e-12)


def test_headline_flops_of_the_named_workloads():
    # 1.522, 83.24 and 330.58 nominal TFLOP per step (C1, C2, C4)
    assert W.config(1).nominal_ns_flops() / 1e12 == pytest.approx(1.522, abs=5e-4)
    assert W.config(2).nominal_ns_flops() / 1e12 == pytest.approx(83.24, abs=5e-3)
    assert W.config(4).nominal_ns_flops() / 1e12 == pytest.approx(330.58, abs=5e-3)


def test_mixed_set_draw():
    wl = W.config(3)
    specs = wl.muon_specs()
    assert len(specs) == 256
    for s in specs:
        m, n = min(s.rows, s.cols), max(s.rows, s.cols)
        assert m in (512, 1024, 2048, 4096) and n // m in (1, 2, 4, 8) and n % m == 0
    assert {s.rows > s.cols for s in specs if s.rows != s.cols} == {True, False}  # tall and wide


def test_traffic_record_follows_the_sources():
    sys.path.insert(0, ROOT)
    import bench

    dig = bench.sources_digest()
    assert len(dig) == 16
    for (workload, prec, phase), (d, fetch, write) in bench.TRAFFIC.items():
        assert fetch > 0 and write > 0
        want = fetch + write if d == dig else None
        assert bench.measured_traffic(workload, prec, phase) == want
    assert bench.measured_traffic("no-such-workload", "bf16", "update") is None
