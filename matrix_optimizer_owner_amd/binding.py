"""ctypes binding of libmfsdp.so (the C ABI in include/mfsdp.h).

Argument marshalling only: every step of the optimizer runs in the HIP
library.  Buffers are passed as integer device addresses (for a torch
tensor, ``t.data_ptr()``); streams as integer ``hipStream_t`` handles (for
torch, ``torch.cuda.current_stream().cuda_stream``).  If the library has not
been built, loading raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmfsdp.so")

F32, BF16 = 0, 1
ROLE_AUTO, ROLE_MUON, ROLE_ADAMW = 0, 1, 2
STEP_DESCRIPTORS_RESIDENT = 1
STATIC_WORKSPACE_BYTES = 64 << 20  # MFSDP_STATIC_WORKSPACE_BYTES

STATUS = {
    0: "MFSDP_OK",
    1: "MFSDP_ERR_INVALID_ARGUMENT",
    2: "MFSDP_ERR_OVERLAP",
    3: "MFSDP_ERR_MISALIGNED",
    4: "MFSDP_ERR_UNSUPPORTED",
    5: "MFSDP_ERR_WORKSPACE_TOO_SMALL",
    6: "MFSDP_ERR_HIP",
    7: "MFSDP_ERR_INTERNAL",
}


class Entry(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("dtype", ctypes.c_int32), ("role", ctypes.c_int32)]


class Hparams(ctypes.Structure):
    _fields_ = [
        ("lr", ctypes.c_float), ("weight_decay", ctypes.c_float), ("momentum", ctypes.c_float),
        ("nesterov", ctypes.c_int32), ("ns_steps", ctypes.c_int32),
        ("ns_a", ctypes.c_float), ("ns_b", ctypes.c_float), ("ns_c", ctypes.c_float), ("ns_eps", ctypes.c_float),
        ("lr_scale_mode", ctypes.c_int32), ("ns_precision", ctypes.c_int32),
        ("adam_lr", ctypes.c_float), ("adam_beta1", ctypes.c_float), ("adam_beta2", ctypes.c_float),
        ("adam_eps", ctypes.c_float), ("adam_weight_decay", ctypes.c_float),
        ("momentum_dtype", ctypes.c_int32),
        ("ns_tile_gram", ctypes.c_int32), ("ns_tile_poly", ctypes.c_int32), ("ns_tile_update", ctypes.c_int32),
        ("guard_bytes", ctypes.c_uint32),
    ]


class EntryInfo(ctypes.Structure):
    _fields_ = [("role", ctypes.c_int32), ("transposed", ctypes.c_int32), ("m", ctypes.c_int64),
                ("n", ctypes.c_int64), ("state_offset", ctypes.c_uint64), ("state_offset2", ctypes.c_uint64),
                ("ns_out_offset", ctypes.c_uint64), ("lr_scale", ctypes.c_float)]


BUFFER_STATE, BUFFER_WORKSPACE = 0, 1


class Region(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_uint64), ("bytes", ctypes.c_uint64), ("buffer", ctypes.c_int32),
                ("entry", ctypes.c_int32)]


class StepArgs(ctypes.Structure):
    _fields_ = [("params", ctypes.c_void_p), ("grads", ctypes.c_void_p), ("state", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64), ("step", ctypes.c_int64),
                ("stream", ctypes.c_void_p), ("ns_out", ctypes.c_void_p), ("flags", ctypes.c_uint32),
                ("events", ctypes.POINTER(ctypes.c_void_p)), ("n_events", ctypes.c_uint32)]


class Tensor(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("dtype", ctypes.c_int32), ("role", ctypes.c_int32)]


class PartitionParams(ctypes.Structure):
    _fields_ = [("n_owners", ctypes.c_int32), ("ns_steps", ctypes.c_int32), ("ns_precision", ctypes.c_int32),
                ("momentum_dtype", ctypes.c_int32), ("mem_cap_bytes", ctypes.c_uint64), ("flop_rate", ctypes.c_double),
                ("byte_rate", ctypes.c_double)]


class TensorPlace(ctypes.Structure):
    _fields_ = [("owner", ctypes.c_int32), ("role", ctypes.c_int32), ("offset", ctypes.c_uint64),
                ("cost", ctypes.c_double), ("mem_bytes", ctypes.c_uint64)]


EXPORTS = (
    "mfsdp_plan_create", "mfsdp_plan_state_bytes", "mfsdp_plan_workspace_bytes", "mfsdp_plan_ns_out_elems",
    "mfsdp_plan_num_events", "mfsdp_plan_num_entries", "mfsdp_plan_entry_info", "mfsdp_plan_regions",
    "mfsdp_owner_step", "mfsdp_owner_step_static", "mfsdp_plan_destroy",
    "mfsdp_owner_partition", "mfsdp_owner_gather", "mfsdp_owner_scatter", "mfsdp_status_string",
    "mfsdp_last_error_message", "mfsdp_probe_mfma_bf16", "mfsdp_probe_hbm",
)

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmfsdp.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m matrix_optimizer_owner_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    u64p = ctypes.POINTER(ctypes.c_uint64)
    lib.mfsdp_plan_create.argtypes = [ctypes.POINTER(Entry), ctypes.c_int64, ctypes.c_uint64,
                                      ctypes.POINTER(Hparams), ctypes.POINTER(P)]
    lib.mfsdp_plan_state_bytes.argtypes = [P, u64p]
    lib.mfsdp_plan_workspace_bytes.argtypes = [P, u64p]
    lib.mfsdp_plan_ns_out_elems.argtypes = [P, u64p]
    lib.mfsdp_plan_num_events.argtypes = [P, ctypes.POINTER(ctypes.c_uint32)]
    lib.mfsdp_plan_num_entries.argtypes = [P, ctypes.POINTER(ctypes.c_int64)]
    lib.mfsdp_plan_entry_info.argtypes = [P, ctypes.c_int64, ctypes.POINTER(EntryInfo)]
    lib.mfsdp_plan_regions.argtypes = [P, ctypes.POINTER(Region), ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
    lib.mfsdp_owner_step.argtypes = [P, ctypes.POINTER(StepArgs)]
    lib.mfsdp_owner_step_static.argtypes = [P, ctypes.POINTER(StepArgs)]
    lib.mfsdp_plan_destroy.argtypes = [P]
    lib.mfsdp_owner_partition.argtypes = [ctypes.POINTER(Tensor), ctypes.c_int64, ctypes.POINTER(PartitionParams),
                                          ctypes.POINTER(TensorPlace), ctypes.POINTER(ctypes.c_double), u64p, u64p]
    vpp = ctypes.POINTER(ctypes.c_void_p)
    lib.mfsdp_owner_gather.argtypes = [P, P, ctypes.c_uint64, P, ctypes.c_uint64, vpp, vpp, vpp]
    lib.mfsdp_owner_scatter.argtypes = [P, vpp, vpp, vpp, P, ctypes.c_uint64, P, ctypes.c_uint64]
    lib.mfsdp_probe_mfma_bf16.argtypes = [P, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, P, P,
                                          ctypes.POINTER(ctypes.c_double)]
    lib.mfsdp_probe_hbm.argtypes = [P, P, ctypes.c_uint64, ctypes.c_int32, P, P]
    lib.mfsdp_status_string.argtypes = [ctypes.c_int]
    lib.mfsdp_status_string.restype = ctypes.c_char_p
    lib.mfsdp_last_error_message.argtypes = []
    lib.mfsdp_last_error_message.restype = ctypes.c_char_p
    for name in EXPORTS:
        if name not in ("mfsdp_status_string", "mfsdp_last_error_message"):
            getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


class MfsdpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def _check(status: int) -> None:
    if status != 0:
        msg = load().mfsdp_last_error_message().decode()
        raise MfsdpError(status, msg)


def make_hparams(**kw) -> Hparams:
    """Hyper-parameters with Muon/AdamW defaults; keyword overrides.
    ``ns_tile=E`` or ``ns_tile=(G, P, U)`` is shorthand for the three
    ns_tile_* fields (the output tile edge of the Gram, polynomial and update
    contractions: 0 = the planner's choice, 128 or 256)."""
    if "ns_tile" in kw:
        t = kw.pop("ns_tile")
        g, p, u = (t, t, t) if isinstance(t, int) else tuple(t)
        kw.update(ns_tile_gram=g, ns_tile_poly=p, ns_tile_update=u)
    d = dict(lr=0.02, weight_decay=0.01, momentum=0.95, nesterov=1, ns_steps=5, ns_a=3.4445, ns_b=-4.7750,
             ns_c=2.0315, ns_eps=1e-7, lr_scale_mode=0, ns_precision=0, adam_lr=0.02, adam_beta1=0.9,
             adam_beta2=0.95, adam_eps=1e-8, adam_weight_decay=0.01, momentum_dtype=0, ns_tile_gram=0,
             ns_tile_poly=0, ns_tile_update=0, guard_bytes=0)
    unknown = set(kw) - set(d)
    if unknown:
        raise KeyError(f"unknown hyper-parameters {sorted(unknown)}")
    d.update(kw)
    ints = {"nesterov", "ns_steps", "lr_scale_mode", "ns_precision", "momentum_dtype", "ns_tile_gram",
            "ns_tile_poly", "ns_tile_update", "guard_bytes"}
    return Hparams(**{k: (int(v) if k in ints else float(v)) for k, v in d.items()})


@dataclass(frozen=True)
class TableEntry:
    offset: int
    rows: int
    cols: int
    dtype: int = BF16
    role: int = ROLE_AUTO


class OwnerPlan:
    """A lowered owner table (mfsdp_plan_t) and its step call."""

    def __init__(self, entries: Sequence[TableEntry], param_bytes: int, hparams: Hparams):
        lib = load()
        arr = (Entry * max(1, len(entries)))()
        for i, e in enumerate(entries):
            arr[i] = Entry(e.offset, e.rows, e.cols, e.dtype, e.role)
        handle = ctypes.c_void_p()
        self.hparams = hparams
        _check(lib.mfsdp_plan_create(arr, len(entries), param_bytes, ctypes.byref(hparams), ctypes.byref(handle)))
        self._h = handle
        self._lib = lib
        self.n_entries = len(entries)

    def _u64(self, fn) -> int:
        v = ctypes.c_uint64()
        _check(fn(self._h, ctypes.byref(v)))
        return v.value

    @property
    def state_bytes(self) -> int:
        return self._u64(self._lib.mfsdp_plan_state_bytes)

    @property
    def workspace_bytes(self) -> int:
        return self._u64(self._lib.mfsdp_plan_workspace_bytes)

    @property
    def ns_out_elems(self) -> int:
        return self._u64(self._lib.mfsdp_plan_ns_out_elems)

    def num_entries(self) -> int:
        v = ctypes.c_int64()
        _check(self._lib.mfsdp_plan_num_entries(self._h, ctypes.byref(v)))
        return v.value

    def entry_info(self, i: int) -> EntryInfo:
        info = EntryInfo()
        _check(self._lib.mfsdp_plan_entry_info(self._h, i, ctypes.byref(info)))
        return info

    def regions(self) -> list:
        """Every state and workspace region of the plan (mfsdp_plan_regions)."""
        n = ctypes.c_int64()
        _check(self._lib.mfsdp_plan_regions(self._h, None, 0, ctypes.byref(n)))
        arr = (Region * max(1, n.value))()
        _check(self._lib.mfsdp_plan_regions(self._h, arr, n.value, ctypes.byref(n)))
        return [arr[k] for k in range(n.value)]

    def num_events(self) -> int:
        v = ctypes.c_uint32()
        _check(self._lib.mfsdp_plan_num_events(self._h, ctypes.byref(v)))
        return v.value

    def step(self, params: int, grads: int, state: int, workspace: int, workspace_bytes: int, step: int,
             stream: int = 0, ns_out: int = 0, flags: int = 0, events: Sequence[int] = ()) -> None:
        ev = (ctypes.c_void_p * len(events))(*events) if events else None
        args = StepArgs(params, grads, state, workspace, workspace_bytes, step, stream or None, ns_out or None, flags,
                        ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)) if ev is not None else None, len(events))
        _check(self._lib.mfsdp_owner_step(self._h, ctypes.byref(args)))

    def step_static(self, params: int, grads: int, state: int, step: int, stream: int = 0, ns_out: int = 0,
                    flags: int = 0, events: Sequence[int] = ()) -> None:
        """mfsdp_owner_step_static: the step on the library's own workspace
        (no allocation; at most STATIC_WORKSPACE_BYTES of workspace)."""
        ev = (ctypes.c_void_p * len(events))(*events) if events else None
        args = StepArgs(params, grads, state, None, 0, step, stream or None, ns_out or None, flags,
                        ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)) if ev is not None else None, len(events))
        _check(self._lib.mfsdp_owner_step_static(self._h, ctypes.byref(args)))

    def _ptrs(self, addrs):
        if addrs is None:
            return None
        if len(addrs) != self.n_entries:
            raise ValueError(f"{len(addrs)} buffers for {self.n_entries} entries")
        return (ctypes.c_void_p * max(1, self.n_entries))(*[a or None for a in addrs])

    def gather(self, params: int, param_bytes: int, state: int, state_bytes: int, tensors=None, state1=None,
               state2=None) -> None:
        """Copy the owner's tensors and state (host buffers at the given
        addresses) out to one host buffer per entry (lists of addresses,
        0 for none; a list may be None)."""
        _check(self._lib.mfsdp_owner_gather(self._h, params or None, param_bytes, state or None, state_bytes,
                                            self._ptrs(tensors), self._ptrs(state1), self._ptrs(state2)))

    def scatter(self, tensors, state1, state2, params: int, param_bytes: int, state: int, state_bytes: int) -> None:
        """Copy per-entry host buffers into the owner's flat host buffers."""
        _check(self._lib.mfsdp_owner_scatter(self._h, self._ptrs(tensors), self._ptrs(state1), self._ptrs(state2),
                                             params or None, param_bytes, state or None, state_bytes))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            self._lib.mfsdp_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


@dataclass(frozen=True)
class Partition:
    """Result of owner_partition: per tensor its owner, resolved role and
    byte offset in that owner's flat parameter buffer, and its model cost and
    memory; per owner the summed cost, memory and parameter bytes."""
    owner: list
    role: list
    offset: list
    cost: list
    mem_bytes: list
    owner_cost: list
    owner_mem_bytes: list
    owner_param_bytes: list

    def table(self, o: int, dtypes: Sequence[int], shapes: Sequence[tuple]) -> list:
        """Owner o's table (input order) as TableEntry rows."""
        return [TableEntry(self.offset[i], shapes[i][0], shapes[i][1], dtypes[i], self.role[i])
                for i in range(len(self.owner)) if self.owner[i] == o]


def owner_partition(shapes: Sequence[tuple], dtypes: Sequence[int], n_owners: int, *, roles: Sequence[int] = None,
                    ns_steps: int = 5, ns_precision: int = 0, mem_cap_bytes: int = 0, flop_rate: float = 1.6e15,
                    byte_rate: float = 5.2e12, momentum_dtype: int = 0) -> Partition:
    """Balance-aware assignment of whole tensors to owners (mfsdp_owner_partition)."""
    lib = load()
    n = len(shapes)
    roles = list(roles) if roles is not None else [ROLE_AUTO] * n
    arr = (Tensor * max(n, 1))(*[Tensor(int(r), int(c), int(dt), int(ro))
                                 for (r, c), dt, ro in zip(shapes, dtypes, roles)])
    pp = PartitionParams(int(n_owners), int(ns_steps), int(ns_precision), int(momentum_dtype), int(mem_cap_bytes),
                         float(flop_rate),
                         float(byte_rate))
    place = (TensorPlace * max(n, 1))()
    oc = (ctypes.c_double * max(int(n_owners), 1))()
    om = (ctypes.c_uint64 * max(int(n_owners), 1))()
    ob = (ctypes.c_uint64 * max(int(n_owners), 1))()
    _check(lib.mfsdp_owner_partition(arr, n, ctypes.byref(pp), place, oc, om, ob))
    return Partition([place[i].owner for i in range(n)], [place[i].role for i in range(n)],
                     [place[i].offset for i in range(n)], [place[i].cost for i in range(n)],
                     [place[i].mem_bytes for i in range(n)], list(oc[:n_owners]), list(om[:n_owners]),
                     list(ob[:n_owners]))


def probe_mfma_bf16(operands: int, operand_bytes: int, blocks: int, iters: int, sink: int, stream: int = 0) -> float:
    """Enqueue the register-only bf16 MFMA loop (mfsdp_probe_mfma_bf16) on
    `stream` over device operands; returns the FLOPs enqueued."""
    lib = load()
    flops = ctypes.c_double()
    _check(lib.mfsdp_probe_mfma_bf16(ctypes.c_void_p(operands), operand_bytes, blocks, iters, ctypes.c_void_p(sink),
                                     ctypes.c_void_p(stream), ctypes.byref(flops)))
    return flops.value


def probe_hbm(dst: int, src: int, nbytes: int, mode: int, sink: int, stream: int = 0) -> None:
    """Enqueue one streaming pass (mfsdp_probe_hbm): mode 0 read, 1 write,
    2 copy."""
    _check(load().mfsdp_probe_hbm(ctypes.c_void_p(dst), ctypes.c_void_p(src), nbytes, mode, ctypes.c_void_p(sink),
                                  ctypes.c_void_p(stream)))
