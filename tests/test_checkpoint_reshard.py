"""Host tests of owner-shard checkpoint resharding (mfsdp_owner_gather /
mfsdp_owner_scatter with mfsdp_owner_partition): whole tensors and their
optimizer state survive owner layout -> full tensors -> another owner count
-> back, bit for bit.  No GPU is needed."""

import numpy as np
import pytest

from matrix_optimizer_owner_amd import binding as B


def _model(rng):
    shapes, dtypes = [], []
    for _ in range(6):
        shapes += [(512, 512), (128, 512), (1536, 512), (512, 1536), (1, 512), (0, 64)]
        dtypes += [B.BF16, B.BF16, B.BF16, B.F32, B.F32, B.BF16]
    shapes += [(300, 70), (70, 300), (1, 1)]
    dtypes += [B.F32, B.BF16, B.F32]
    return shapes, dtypes


class Owners:
    """Host buffers of every owner of a partition: flat params and state."""

    def __init__(self, shapes, dtypes, n_owners, momentum_dtype=B.F32):
        self.shapes, self.dtypes, self.mdt = shapes, dtypes, momentum_dtype
        self.part = B.owner_partition(shapes, dtypes, n_owners, momentum_dtype=momentum_dtype)
        self.tables = [self.part.table(o, dtypes, shapes) for o in range(n_owners)]
        hp = B.make_hparams(momentum_dtype=momentum_dtype)
        self.plans = [B.OwnerPlan(t, self.part.owner_param_bytes[o], hp) for o, t in enumerate(self.tables)]
        self.params = [np.zeros(max(1, self.part.owner_param_bytes[o]), np.uint8) for o in range(n_owners)]
        self.state = [np.zeros(max(1, p.state_bytes), np.uint8) for p in self.plans]
        self.index = [[i for i in range(len(shapes)) if self.part.owner[i] == o] for o in range(n_owners)]

    def close(self):
        for p in self.plans:
            p.close()

    def _bufs(self, o, full):
        """Per-entry addresses of owner o into the full checkpoint."""
        t = [full["param"][i].ctypes.data if full["param"][i].size else 0 for i in self.index[o]]
        s1 = [full["s1"][i].ctypes.data if full["s1"][i] is not None and full["s1"][i].size else 0 for i in self.index[o]]
        s2 = [full["s2"][i].ctypes.data if full["s2"][i] is not None and full["s2"][i].size else 0 for i in self.index[o]]
        return t, s1, s2

    def gather(self):
        full = empty_checkpoint(self.shapes, self.dtypes, self.part.role, self.mdt)
        for o, plan in enumerate(self.plans):
            t, s1, s2 = self._bufs(o, full)
            plan.gather(self.params[o].ctypes.data, self.params[o].size, self.state[o].ctypes.data,
                        self.state[o].size, t, s1, s2)
        return full

    def scatter(self, full):
        for o, plan in enumerate(self.plans):
            t, s1, s2 = self._bufs(o, full)
            plan.scatter(t, s1, s2, self.params[o].ctypes.data, self.params[o].size, self.state[o].ctypes.data,
                         self.state[o].size)


def empty_checkpoint(shapes, dtypes, roles, momentum_dtype=B.F32):
    param = [np.zeros(r * c * (2 if dt == B.BF16 else 4), np.uint8) for (r, c), dt in zip(shapes, dtypes)]
    # Muon momentum in the plan's momentum type (bf16 as raw 16-bit words), AdamW moments fp32
    s1 = [(np.zeros(r * c, np.uint16) if ro == B.ROLE_MUON and momentum_dtype == B.BF16 else np.zeros(r * c, np.float32))
          if r * c else None for (r, c), ro in zip(shapes, roles)]
    s2 = [np.zeros(r * c, np.float32) if r * c and ro == B.ROLE_ADAMW else None
          for (r, c), ro in zip(shapes, roles)]
    return {"param": param, "s1": s1, "s2": s2}


def random_checkpoint(rng, shapes, dtypes, roles, momentum_dtype=B.F32):
    full = empty_checkpoint(shapes, dtypes, roles, momentum_dtype)
    for i in range(len(shapes)):
        full["param"][i][:] = rng.integers(0, 256, full["param"][i].size, dtype=np.uint8)
        for k in ("s1", "s2"):
            if full[k][i] is not None:
                # arbitrary bit patterns, NaN payloads and signed zeros included
                bits = rng.integers(0, 2 ** 32, full[k][i].size, dtype=np.uint64)
                full[k][i][:] = (bits.astype(np.uint16) if full[k][i].dtype == np.uint16
                                 else bits.astype(np.uint32).view(np.float32))
    return full


def _same(a, b):
    for k in ("param", "s1", "s2"):
        for x, y in zip(a[k], b[k]):
            if x is None or y is None:
                assert x is None and y is None
            else:
                assert x.view(np.uint8).tobytes() == y.view(np.uint8).tobytes()


@pytest.mark.parametrize("old,new,mdt", [(4, 3, B.F32), (1, 5, B.F32), (6, 2, B.F32), (3, 5, B.BF16)])
def test_reshard_round_trip_bit_exact(old, new, mdt):
    rng = np.random.default_rng(old * 10 + new)
    shapes, dtypes = _model(rng)
    a = Owners(shapes, dtypes, old, mdt)
    b = Owners(shapes, dtypes, new, mdt)
    c = Owners(shapes, dtypes, old, mdt)
    try:
        ckpt = random_checkpoint(rng, shapes, dtypes, a.part.role, mdt)
        a.scatter(ckpt)
        full1 = a.gather()
        _same(full1, ckpt)
        b.scatter(full1)             # another owner count
        full2 = b.gather()
        _same(full2, ckpt)
        c.scatter(full2)             # back to the first count: the same flat buffers
        for o in range(old):
            assert c.params[o].tobytes() == a.params[o].tobytes()
            assert c.state[o].tobytes() == a.state[o].tobytes()
    finally:
        a.close(), b.close(), c.close()


def test_state_lands_at_the_plans_offsets():
    """A gathered momentum / moment is the plan's state region of that entry."""
    rng = np.random.default_rng(3)
    shapes, dtypes = _model(rng)
    own = Owners(shapes, dtypes, 2)
    try:
        ckpt = random_checkpoint(rng, shapes, dtypes, own.part.role)
        own.scatter(ckpt)
        for o, plan in enumerate(own.plans):
            for k, i in enumerate(own.index[o]):
                info = plan.entry_info(k)
                numel = shapes[i][0] * shapes[i][1]
                if numel == 0:
                    continue
                got = own.state[o][info.state_offset:info.state_offset + 4 * numel]
                assert got.tobytes() == ckpt["s1"][i].tobytes()
                if info.role == B.ROLE_ADAMW:
                    got2 = own.state[o][info.state_offset2:info.state_offset2 + 4 * numel]
                    assert got2.tobytes() == ckpt["s2"][i].tobytes()
                off = own.part.offset[i]
                assert own.params[o][off:off + ckpt["param"][i].size].tobytes() == ckpt["param"][i].tobytes()
    finally:
        own.close()


def test_gather_scatter_errors():
    plan = B.OwnerPlan([B.TableEntry(0, 4, 4), B.TableEntry(256, 1, 8, B.F32)], 512, B.make_hparams())
    try:
        p = np.zeros(512, np.uint8)
        st = np.zeros(plan.state_bytes, np.uint8)
        t = [np.zeros(32, np.uint8), np.zeros(32, np.uint8)]
        addrs = [x.ctypes.data for x in t]
        with pytest.raises(B.MfsdpError) as e:          # param buffer too small
            plan.gather(p.ctypes.data, 100, st.ctypes.data, st.size, addrs)
        assert e.value.status == 1
        with pytest.raises(B.MfsdpError) as e:          # state buffer too small
            plan.gather(p.ctypes.data, p.size, st.ctypes.data, st.size - 4, None, addrs)
        assert e.value.status == 1
        with pytest.raises(B.MfsdpError) as e:          # a needed per-tensor buffer missing
            plan.gather(p.ctypes.data, p.size, st.ctypes.data, st.size, [addrs[0], 0])
        assert e.value.status == 1
        with pytest.raises(B.MfsdpError) as e:          # the owner buffer missing
            plan.scatter(addrs, None, None, 0, p.size, st.ctypes.data, st.size)
        assert e.value.status == 1
        plan.gather(p.ctypes.data, p.size, 0, 0, addrs)  # parameters only
    finally:
        plan.close()
