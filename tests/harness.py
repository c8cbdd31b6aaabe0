"""Test harness: run the HIP owner step through the C ABI on seeded buffers,
read every buffer back, and compare with the fp64 oracle.

The oracle is teacher-forced: step t starts from the state the GPU stored
after step t-1, read back from the device.  Criteria (per matrix / tensor):

* O (the Newton-Schulz output, exported in fp32 through ns_out) against the
  oracle's O: relative Frobenius error <= 1e-4 on the fp32 path and <= 3e-2
  on the bf16 path, and on the bf16 path every sorted singular value within
  0.05 of the oracle's;
* parameters: the stored W equals RNE(W (1 - lr wd) - lr scale O_gpu) within
  one unit in the last place of the storage type plus one fp32 ulp of W and
  one of lr scale O (the update arithmetic, given the exported O);
* momentum: relative error <= 1e-6 (one fp32 rounding); stored in bf16
  (momentum_dtype): within half a bf16 ulp of the oracle's value plus 1e-6
  of the larger operand (beta m or g);
* AdamW tail: relative Frobenius error <= 1e-6 on W, m and v (fp32 tails;
  for W relative to the larger of the result and the update's operands);
  bf16 tails: within half a bf16 ulp of the oracle's W plus 1e-6 of the
  larger operand of the update (the fp32 error before the rounding).
"""

from __future__ import annotations

import math
import sys
from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

from matrix_optimizer_owner_amd import binding as B
from matrix_optimizer_owner_amd import workloads as W
from oracle import muon_oracle as orc

DT = {"bf16": B.BF16, "f32": B.F32}
ROLE = {"auto": B.ROLE_AUTO, "muon": B.ROLE_MUON, "adamw": B.ROLE_ADAMW}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bytes_to_f64(u8: np.ndarray, off: int, rows: int, cols: int, dtype: str) -> np.ndarray:
    n = rows * cols
    if dtype == "bf16":
        raw = u8[off:off + 2 * n].view(np.uint16).astype(np.uint32) << np.uint32(16)
        return raw.view(np.float32).astype(np.float64).reshape(rows, cols)
    return u8[off:off + 4 * n].view(np.float32).astype(np.float64).reshape(rows, cols)


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage type at |x| (bf16: 8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    a = np.maximum(a, np.finfo(np.float32).tiny)
    e = np.floor(np.log2(a))
    return np.exp2(e - (7 if dtype == "bf16" else 23))


def oracle_hparams(hp: Dict[str, float]) -> orc.Hparams:
    f = orc.f32
    return orc.Hparams(
        lr=f(hp["lr"]), weight_decay=f(hp["weight_decay"]), momentum=f(hp["momentum"]),
        nesterov=bool(hp["nesterov"]), ns_steps=int(hp["ns_steps"]), ns_a=f(hp["ns_a"]), ns_b=f(hp["ns_b"]),
        ns_c=f(hp["ns_c"]), ns_eps=f(hp["ns_eps"]), lr_scale_mode=int(hp["lr_scale_mode"]),
        adam_lr=f(hp["adam_lr"]), adam_beta1=f(hp["adam_beta1"]), adam_beta2=f(hp["adam_beta2"]),
        adam_eps=f(hp["adam_eps"]), adam_weight_decay=f(hp["adam_weight_decay"]))


class DeviceRun:
    """One workload's plan and device buffers."""

    def __init__(self, wl: W.Workload, hp_overrides=None, device="cuda"):
        import torch

        self.torch = torch
        self.wl = wl
        self.hp = dict(wl.hparams, **(hp_overrides or {}))
        self.offs, self.pbytes = wl.layout()
        entries = [B.TableEntry(o, s.rows, s.cols, DT[s.dtype], ROLE[s.role]) for o, s in zip(self.offs, wl.specs)]
        self.plan = B.OwnerPlan(entries, self.pbytes, B.make_hparams(**self.hp))
        self.info = [self.plan.entry_info(i) for i in range(len(wl.specs))]
        u8 = torch.uint8
        self.params = torch.zeros(self.pbytes, dtype=u8, device=device)
        self.grads = torch.zeros(self.pbytes, dtype=u8, device=device)
        self.state = torch.zeros(max(self.plan.state_bytes, 256), dtype=u8, device=device)
        self.ws_bytes = max(self.plan.workspace_bytes, 256)
        self.ws = torch.zeros(self.ws_bytes, dtype=u8, device=device)
        self.ns_out = torch.zeros(max(self.plan.ns_out_elems, 4), dtype=torch.float32, device=device)
        self.steps_done = 0

    def fill(self, step: int, params_too: bool) -> None:
        W.fill(self.wl, step, self.params, self.grads, params_too=params_too)

    def run(self, step: int, ns_out: bool = True, flags: int = 0) -> None:
        t = self.torch
        self.plan.step(self.params.data_ptr(), self.grads.data_ptr(), self.state.data_ptr(), self.ws.data_ptr(),
                       self.ws_bytes, step, stream=t.cuda.current_stream().cuda_stream,
                       ns_out=self.ns_out.data_ptr() if ns_out else 0, flags=flags)

    def host(self) -> Dict[str, np.ndarray]:
        self.torch.cuda.synchronize()
        return {"params": self.params.cpu().numpy(), "grads": self.grads.cpu().numpy(),
                "state": self.state.cpu().numpy(), "ns_out": self.ns_out.cpu().numpy()}

    # -- per-entry device reads (no full-buffer copies) --
    def dev_entry(self, i: int, what: str) -> np.ndarray:
        """One entry of a device buffer as fp64: what in {"param", "grad",
        "state", "state2", "o"}."""
        t = self.torch
        s = self.wl.specs[i]
        if what in ("param", "grad"):
            buf = self.params if what == "param" else self.grads
            off, nb = self.offs[i], s.numel * s.itemsize
            raw = buf[off:off + nb]
            v = raw.view(t.bfloat16 if s.dtype == "bf16" else t.float32)
        elif what in ("state", "state2"):
            off = self.info[i].state_offset2 if what == "state2" else self.info[i].state_offset
            if self.momentum_bf16(i) and what == "state":
                v = self.state[off:off + 2 * s.numel].view(t.bfloat16)
            else:
                v = self.state[off:off + 4 * s.numel].view(t.float32)
        else:
            off = self.info[i].ns_out_offset
            v = self.ns_out[off:off + s.numel]
        return v.float().cpu().numpy().astype(np.float64).reshape(s.rows, s.cols)

    def snapshot_entries(self, idxs, what_list=("param", "grad", "state")):
        self.torch.cuda.synchronize()
        return {(i, w): self.dev_entry(i, w) for i in idxs for w in what_list}

    def free(self) -> None:
        for name in ("params", "grads", "state", "ws", "ns_out"):
            setattr(self, name, None)
        self.torch.cuda.empty_cache()

    # -- per-entry views of host copies --
    def param(self, snap, i) -> np.ndarray:
        s = self.wl.specs[i]
        return bytes_to_f64(snap["params"], self.offs[i], s.rows, s.cols, s.dtype)

    def grad(self, snap, i) -> np.ndarray:
        s = self.wl.specs[i]
        return bytes_to_f64(snap["grads"], self.offs[i], s.rows, s.cols, s.dtype)

    def momentum_bf16(self, i) -> bool:
        """Entry i is a Muon matrix whose momentum is stored in bf16."""
        return self.info[i].role == B.ROLE_MUON and int(self.hp.get("momentum_dtype", 0)) == B.BF16

    def state_arr(self, snap, i, second=False) -> np.ndarray:
        s = self.wl.specs[i]
        off = self.info[i].state_offset2 if second else self.info[i].state_offset
        return bytes_to_f64(snap["state"], off, s.rows, s.cols, "bf16" if self.momentum_bf16(i) and not second else "f32")

    def o_gpu(self, snap, i) -> np.ndarray:
        s = self.wl.specs[i]
        off = self.info[i].ns_out_offset
        return snap["ns_out"][off:off + s.numel].astype(np.float64).reshape(s.rows, s.cols)


@dataclass
class EntryReport:
    name: str
    role: str
    metrics: Dict[str, float] = field(default_factory=dict)
    failures: List[str] = field(default_factory=list)


def sigma_check(o_gpu: np.ndarray, o_orc: np.ndarray) -> float:
    """max |sigma_i(O_gpu) - sigma_i(O_orc)| over sorted spectra (full SVD
    when min dim <= 2048, else the Weyl bound ||O_gpu - O_orc||_2 from power
    iteration, falling back to eigvalsh of O O^T)."""
    m = min(o_gpu.shape)
    if m <= 2048:
        s1 = np.sort(np.linalg.svd(o_gpu, compute_uv=False))
        s2 = np.sort(np.linalg.svd(o_orc, compute_uv=False))
        return float(np.max(np.abs(s1 - s2)))
    d = o_gpu - o_orc
    v = np.random.default_rng(0).standard_normal(d.shape[1])
    for _ in range(60):
        v = d.T @ (d @ v)
        v /= np.linalg.norm(v)
    bound = float(np.linalg.norm(d @ v))
    if bound <= 0.05:
        return bound
    def spec(o):
        g = o @ o.T if o.shape[0] <= o.shape[1] else o.T @ o
        return np.sqrt(np.clip(np.sort(np.linalg.eigvalsh(g)), 0, None))
    return float(np.max(np.abs(spec(o_gpu) - spec(o_orc))))


def check_step(run: DeviceRun, before, after, step: int, entries=None, sigma=True) -> List[EntryReport]:
    """Compare one GPU step (host copies before/after) with the oracle."""
    hp = oracle_hparams(run.hp)
    prec = int(run.hp["ns_precision"])
    o_tol = 1e-4 if prec == 1 else 3e-2
    reports = []
    idxs = range(len(run.wl.specs)) if entries is None else entries
    for i in idxs:
        s = run.wl.specs[i]
        inf = run.info[i]
        rep = EntryReport(s.name, {1: "muon", 2: "adamw", -1: "empty"}[inf.role])
        reports.append(rep)
        if inf.role == -1:
            continue
        w0, g = run.param(before, i), run.grad(before, i)
        w1 = run.param(after, i)
        if inf.role == B.ROLE_MUON:
            m0 = run.state_arr(before, i)
            w_orc, m_orc, o_orc = orc.muon_matrix_step(w0, g, m0, hp)
            o_gpu = run.o_gpu(after, i)
            nrm = np.linalg.norm(o_orc)
            rel = np.linalg.norm(o_gpu - o_orc) / nrm if nrm > 0 else np.linalg.norm(o_gpu)
            rep.metrics["o_rel"] = float(rel)
            if not rel <= o_tol:
                rep.failures.append(f"O relative error {rel:.3e} > {o_tol}")
            if prec == 0 and sigma and nrm > 0:
                ds = sigma_check(o_gpu, o_orc)
                rep.metrics["sigma_max_diff"] = ds
                if not ds <= 0.05:
                    rep.failures.append(f"singular values differ by {ds:.3e} > 0.05")
            # parameter update arithmetic given the exported O
            scale = orc.lr_shape_scale(s.rows, s.cols, hp.lr_scale_mode)
            w_ref = w0 * (1.0 - hp.lr * hp.weight_decay) - hp.lr * scale * o_gpu
            w_ref_st = orc.round_to_dtype(w_ref, s.dtype)
            # The GPU forms t = W - (lr wd) W with one fp32 rounding (at most
            # half an fp32 ulp of W), then t - step O with step = lr scale
            # rounded once to fp32 (relative error 2^-24, at most one fp32 ulp
            # of the step term), and rounds to storage.  Allowed: one storage
            # ulp of the result plus one fp32 ulp of W plus one of the step
            # term (the fp32 terms matter for fp32 parameters and when the two
            # terms cancel).
            step_term = np.abs(hp.lr * scale * o_gpu)
            tol = ulp(w_ref_st, s.dtype) + ulp(w0, "f32") + ulp(step_term, "f32")
            werr = np.abs(w1 - w_ref_st) / tol
            rep.metrics["w_err_over_tol"] = float(werr.max())
            if not werr.max() <= 1.0:
                rep.failures.append(f"param differs by {werr.max():.2f} ulp from the update of O_gpu")
            # against the full oracle (informational, plus a loose bound)
            full = np.abs(w1 - orc.round_to_dtype(w_orc, s.dtype))
            rep.metrics["w_vs_oracle_max_abs"] = float(full.max())
            m1 = run.state_arr(after, i)
            if run.momentum_bf16(i):
                # one fp32 FMA, then RNE to bf16: RNE of the oracle's value
                # except within 1e-6 of a bf16 rounding midpoint, relative to
                # the larger operand (beta m or g: the fp32 error scales with
                # them, not with a result that may cancel)
                scale = np.maximum(np.abs(hp.momentum * m0), np.abs(g))
                tol = 0.5 * ulp(m_orc, "bf16") + 1e-6 * np.maximum(scale, np.abs(m_orc))
                bad = int((np.abs(m1 - m_orc) > tol).sum())
                rep.metrics["mom_bf16_bad"] = bad
                if bad:
                    rep.failures.append(f"bf16 momentum: {bad} elements off RNE(oracle)")
            else:
                mrel = np.max(np.abs(m1 - m_orc)) / max(np.max(np.abs(m_orc)), 1e-30)
                rep.metrics["mom_rel"] = float(mrel)
                if not mrel <= 1e-6:
                    rep.failures.append(f"momentum relative error {mrel:.3e} > 1e-6")
        else:
            m0, v0 = run.state_arr(before, i), run.state_arr(before, i, True)
            w_orc, m_orc, v_orc = orc.adamw_step(w0, g, m0, v0, step, hp)
            m1, v1 = run.state_arr(after, i), run.state_arr(after, i, True)
            for nm, got, want in (("m", m1, m_orc), ("v", v1, v_orc)):
                d = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
                rep.metrics[f"adam_{nm}_rel"] = float(d)
                if not d <= 1e-6:
                    rep.failures.append(f"AdamW {nm} relative error {d:.3e} > 1e-6")
            if s.dtype == "f32":
                # relative to the larger of the result and the update's
                # operands (W and lr m_hat / (sqrt(v_hat) + eps)): for a
                # tensor whose W and step nearly cancel (a scalar, say) the
                # result-relative error of exact fp32 arithmetic is unbounded
                m_hat = m_orc / (1.0 - hp.adam_beta1 ** step)
                v_hat = v_orc / (1.0 - hp.adam_beta2 ** step)
                step_term = hp.adam_lr * np.abs(m_hat) / (np.sqrt(v_hat) + hp.adam_eps)
                ref = max(np.linalg.norm(w_orc), np.linalg.norm(w0), np.linalg.norm(step_term), 1e-300)
                d = np.linalg.norm(w1 - w_orc) / ref
                rep.metrics["adam_w_rel"] = float(d)
                if not d <= 1e-6:
                    rep.failures.append(f"AdamW W relative error {d:.3e} > 1e-6")
            else:
                # RNE of the oracle's W except within 1e-6 of a bf16 rounding
                # midpoint, relative to the larger operand of the update (W or
                # lr m_hat / (sqrt(v_hat) + eps)): the kernel's fp32 error
                # scales with them, and the two may cancel
                m_hat = m_orc / (1.0 - hp.adam_beta1 ** step)
                v_hat = v_orc / (1.0 - hp.adam_beta2 ** step)
                step_term = hp.adam_lr * np.abs(m_hat) / (np.sqrt(v_hat) + hp.adam_eps)
                scale = np.maximum(np.maximum(np.abs(w0), step_term), np.abs(w_orc))
                tol = 0.5 * ulp(w_orc, "bf16") + 1e-6 * scale
                bad = np.abs(w1 - w_orc) > tol
                rep.metrics["adam_w_bf16_bad"] = int(bad.sum())
                if bad.any():
                    rep.failures.append(f"AdamW bf16 W: {int(bad.sum())} elements off RNE(oracle)")
    return reports


def assert_reports(reports: List[EntryReport], label: str) -> None:
    bad = [r for r in reports if r.failures]
    for r in reports:
        if r.metrics:
            say(f"  [{label}] {r.name:>28s} {r.role:5s} " + " ".join(f"{k}={v:.3g}" for k, v in r.metrics.items()))
    assert not bad, "; ".join(f"{r.name}: {', '.join(r.failures)}" for r in bad)
