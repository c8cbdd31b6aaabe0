"""Host tests of the balance-aware owner planner (mfsdp_owner_partition):
its cost and memory model, optimality against brute force on small
instances, the memory cap, the owners' tables as plans, balance on whole
models, determinism and argument errors.  No GPU is needed."""

import itertools
import math

import numpy as np
import pytest

from matrix_optimizer_owner_amd import binding as B

FLOP, BYTE = 1.6e15, 5.2e12


def _region(x):
    return (x + 255) // 256 * 256


def _model(rows, cols, dtype, role=B.ROLE_AUTO, ns_steps=5, es_ns=2, em=4):
    """Cost (s) and memory (bytes) of one tensor by the model stated in mfsdp.h."""
    es = 2 if dtype == B.BF16 else 4
    numel = rows * cols
    muon = role == B.ROLE_MUON or (role == B.ROLE_AUTO and rows > 1 and cols > 1)
    if numel == 0:
        muon = False
    if muon:
        m, n = min(rows, cols), max(rows, cols)
        mp, np_ = -(-m // 256) * 256, -(-n // 256) * 256
        cost = ns_steps * (4 * m * m * n + 2 * m ** 3) / FLOP + numel * (3 * es + 2 * em + es_ns) / BYTE
        mem = 2 * _region(numel * es) + _region(numel * em) + 2 * _region(mp * np_ * es_ns) + 2 * _region(mp * mp * es_ns)
    else:
        cost = numel * (3 * es + 16) / BYTE
        mem = 2 * _region(numel * es) + 2 * _region(numel * 4)
    return cost, mem, muon


def _random_instance(rng, n):
    dims = [256, 512, 768, 1024, 1536, 2048, 4096]
    shapes, dtypes = [], []
    for _ in range(n):
        if rng.random() < 0.2:
            shapes.append((1, int(rng.choice(dims))))
            dtypes.append(B.F32)
        else:
            shapes.append((int(rng.choice(dims)), int(rng.choice(dims))))
            dtypes.append(B.BF16)
    return shapes, dtypes


def test_cost_and_memory_model():
    shapes = [(4096, 14336), (14336, 4096), (1024, 4096), (768, 768), (1, 4096), (0, 128), (300, 70)]
    dtypes = [B.BF16, B.BF16, B.BF16, B.F32, B.F32, B.BF16, B.F32]
    p = B.owner_partition(shapes, dtypes, 3, flop_rate=FLOP, byte_rate=BYTE)
    for i, (sh, dt) in enumerate(zip(shapes, dtypes)):
        cost, mem, muon = _model(*sh, dt)
        assert p.role[i] == (B.ROLE_MUON if muon else B.ROLE_ADAMW)
        assert math.isclose(p.cost[i], cost, rel_tol=1e-12), (i, p.cost[i], cost)
        assert p.mem_bytes[i] == mem, (i, p.mem_bytes[i], mem)
    # fp32 Newton-Schulz buffers and another step count
    p = B.owner_partition([(512, 1024)], [B.BF16], 1, ns_steps=3, ns_precision=1)
    cost, mem, _ = _model(512, 1024, B.BF16, ns_steps=3, es_ns=4)
    assert math.isclose(p.cost[0], cost, rel_tol=1e-12) and p.mem_bytes[0] == mem
    # bf16 momentum: 2 B per Muon element of state, 4 B less traffic
    p = B.owner_partition(shapes, dtypes, 3, flop_rate=FLOP, byte_rate=BYTE, momentum_dtype=B.BF16)
    for i, (sh, dt) in enumerate(zip(shapes, dtypes)):
        cost, mem, _ = _model(*sh, dt, em=2)
        assert math.isclose(p.cost[i], cost, rel_tol=1e-12) and p.mem_bytes[i] == mem, i


@pytest.mark.parametrize("n_owners", [2, 3])
def test_brute_force_optimality_small(n_owners):
    """Largest owner cost against the optimum by enumeration (n_owners^n
    assignments): never above the longest-processing-time bound, and at the
    optimum on most random instances."""
    rng = np.random.default_rng(100 + n_owners)
    optimal, trials = 0, 40
    for trial in range(trials):
        n = int(rng.integers(3, 9))
        shapes, dtypes = _random_instance(rng, n)
        p = B.owner_partition(shapes, dtypes, n_owners)
        costs = np.array(p.cost)
        got = max(p.owner_cost)
        best = min(max(np.bincount(np.array(a), weights=costs, minlength=n_owners))
                   for a in itertools.product(range(n_owners), repeat=n))
        bound = (4.0 / 3.0 - 1.0 / (3 * n_owners)) * best
        assert got <= bound * (1 + 1e-12), (trial, shapes, got, best)
        assert got >= best * (1 - 1e-12)
        optimal += got <= best * (1 + 1e-12)
    assert optimal >= 0.8 * trials, optimal


def test_memory_cap():
    rng = np.random.default_rng(7)
    shapes, dtypes = _random_instance(rng, 24)
    free = B.owner_partition(shapes, dtypes, 4)
    total = sum(free.mem_bytes)
    cap = int(max(total / 4 * 1.15, max(free.mem_bytes)))
    p = B.owner_partition(shapes, dtypes, 4, mem_cap_bytes=cap)
    assert max(p.owner_mem_bytes) <= cap
    assert sum(p.owner_mem_bytes) == total
    for o in range(4):
        assert p.owner_mem_bytes[o] == sum(m for m, ow in zip(p.mem_bytes, p.owner) if ow == o)
    # a tensor larger than the cap, and no room left
    with pytest.raises(B.MfsdpError) as e:
        B.owner_partition(shapes, dtypes, 4, mem_cap_bytes=max(free.mem_bytes) - 1)
    assert e.value.status == 4
    with pytest.raises(B.MfsdpError) as e:
        B.owner_partition(shapes, dtypes, 2, mem_cap_bytes=int(total / 2 * 0.9))
    assert e.value.status == 4


def _llama_layers(layers, d, kv, ffn):
    shapes, dtypes = [], []
    for _ in range(layers):
        shapes += [(d, d), (kv, d), (kv, d), (d, d), (ffn, d), (ffn, d), (d, ffn), (1, d), (1, d)]
        dtypes += [B.BF16] * 7 + [B.F32] * 2
    shapes.append((1, d))
    dtypes.append(B.F32)
    return shapes, dtypes


@pytest.mark.parametrize("model,n_owners,mdt", [("llama3-8b", 8, 0), ("llama3-70b", 8, 0), ("llama3-8b", 6, 0),
                                                ("llama3-8b", 8, 1)])
def test_whole_model_balance_and_tables(model, n_owners, mdt):
    """Every Muon matrix of a Llama-3 model over n_owners: owner costs within
    1% of each other's mean, and each owner's table (input order, returned
    offsets) is a plan mfsdp_plan_create accepts whose state, workspace and
    two copies of the parameter bytes equal the modelled memory plus the
    plan's descriptor region."""
    if model == "llama3-8b":
        shapes, dtypes = _llama_layers(32, 4096, 1024, 14336)
    else:
        shapes, dtypes = _llama_layers(80, 8192, 1024, 28672)
    p = B.owner_partition(shapes, dtypes, n_owners, momentum_dtype=mdt)
    mean = sum(p.owner_cost) / n_owners
    assert max(p.owner_cost) <= 1.01 * mean, (max(p.owner_cost), mean)
    hp = B.make_hparams(momentum_dtype=mdt)
    for o in range(n_owners):
        table = p.table(o, dtypes, shapes)
        offs = [e.offset for e in table]
        assert offs == sorted(offs) and all(x % 256 == 0 for x in offs)
        plan = B.OwnerPlan(table, p.owner_param_bytes[o], hp)
        try:
            used = 2 * p.owner_param_bytes[o] + plan.state_bytes + plan.workspace_bytes
            assert p.owner_mem_bytes[o] <= used <= p.owner_mem_bytes[o] * 1.001 + (1 << 20), (o, used)
        finally:
            plan.close()


def test_deterministic_and_empty():
    shapes, dtypes = _llama_layers(8, 2048, 512, 5632)
    a = B.owner_partition(shapes, dtypes, 5)
    b = B.owner_partition(shapes, dtypes, 5)
    assert a == b
    e = B.owner_partition([], [], 3)
    assert e.owner == [] and e.owner_cost == [0.0, 0.0, 0.0] and e.owner_param_bytes == [0, 0, 0]
    one = B.owner_partition([(4096, 4096)], [B.BF16], 4)
    assert one.owner == [0] and one.owner_cost[1:] == [0.0, 0.0, 0.0]


def test_argument_errors():
    def status(**kw):
        args = dict(shapes=[(64, 64)], dtypes=[B.BF16], n_owners=2)
        args.update(kw)
        try:
            B.owner_partition(args.pop("shapes"), args.pop("dtypes"), args.pop("n_owners"), **args)
            return 0
        except B.MfsdpError as err:
            return err.status
    assert status(n_owners=0) == 1
    assert status(shapes=[(-1, 4)]) == 1
    assert status(flop_rate=0.0) == 1
    assert status(byte_rate=float("inf")) == 1
    assert status(ns_steps=-1) == 1
    assert status(momentum_dtype=2) == 4
    assert status(ns_precision=2) == 4
    assert status(dtypes=[7]) == 4
    assert status(roles=[9]) == 4
    assert status(shapes=[(1 << 23, 2)]) == 4
