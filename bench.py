#!/usr/bin/env python3
"""Owner-step benchmark on one MI355X.

One step = one call of mfsdp_owner_step over the whole owner buffer: AdamW
tail, momentum/cast/norm, and ns_steps x (Gram, polynomial, update) with the
fused parameter update - every row of the hot path.  Inputs are seeded,
synthetic and resident in HBM before the timed region.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config I] [--gpus 1]

--config selects the workload (0 single 256x512 fp32, 1 GPT-2-small owner
buffer, 2 Llama-3-8B owner share, 3 mixed 256-matrix stress (default: the
largest workload in Newton-Schulz FLOPs), 4 Llama-3-70B owner share, 5 a
tail-only buffer of 268 M fp32 elements that measures the AdamW kernel
against HBM bandwidth).  --copy-probe-gib G instead runs a plain device copy
of G GiB (used to scale the HBM byte counters of rocprofv3).

Every step, warm-up included, reads its own seeded gradient: up to --steps
gradient buffers (at most --grad-pool-gb of them) are generated before the
timed region, and step k reads buffer k modulo their number.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "Muon owner-step latency (ms) + NS TFLOP/s and % bf16 MFMA peak, 1×MI355X"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}  # dense MFMA, MI355X public figures
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t handles through libamdhip64 (timing only)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n: int):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.lib.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def elapsed_ms(self, a: int, b: int) -> float:
        v = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(v.value)

    def destroy(self, evs) -> None:
        for e in evs:
            self.lib.hipEventDestroy(ctypes.c_void_p(e))


def copy_probe(gib: float) -> None:
    import torch

    n = int(gib * (1 << 30))
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}))


def cpu_baseline(wl, budget_s: float):
    """Time the fp64 oracle on a bounded sample of this workload's matrices
    (host cores), extrapolated to the whole step by nominal NS FLOPs."""
    import numpy as np

    from oracle import muon_oracle as orc

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"] or [0])
    except Exception:
        cores = 0
    cores = cores or os.cpu_count()
    hp = orc.Hparams(ns_steps=int(wl.hparams.get("ns_steps", 5)))
    specs = wl.muon_specs()
    steps = hp.ns_steps
    if not specs:
        return cpu_baseline_tail(wl, hp, budget_s, cores)

    def flops(s):
        m, n = min(s.rows, s.cols), max(s.rows, s.cols)
        return steps * (4.0 * m * m * n + 2.0 * m ** 3)

    # one matrix of each distinct shape, cheapest first, while the estimated
    # total stays within 1.5x the budget (the rate estimated at 0.3 TFLOP/s of
    # fp64 until the first measurement), so that a workload of few, large
    # shapes still gets a sample of about the budget
    seen, sample = set(), []
    for s in sorted(specs, key=flops):
        key = (s.rows, s.cols)
        if key not in seen:
            seen.add(key)
            sample.append(s)
    rng = np.random.default_rng(0)
    t_used, f_used, names = 0.0, 0.0, []
    rate = 0.3e12
    for s in sample:
        if t_used > 0 and t_used + flops(s) / rate > 1.5 * budget_s:
            continue
        w = rng.standard_normal((s.rows, s.cols)) * 0.02
        g = rng.standard_normal((s.rows, s.cols)) * s.grad_std
        m = np.zeros_like(g)
        t0 = time.perf_counter()
        orc.muon_matrix_step(w, g, m, hp)
        dt = time.perf_counter() - t0
        t_used += dt
        f_used += flops(s)
        rate = f_used / t_used
        names.append(f"{s.rows}x{s.cols}")
    total = wl.nominal_ns_flops()
    est_ms = t_used * (total / f_used) * 1e3 if f_used else None
    return {
        "value": est_ms,
        "unit": "ms",
        "cores": int(cores),
        "kind": "oracle",
        "sample": (f"fp64 oracle Muon step on one matrix of each of {len(names)} shapes ({', '.join(names)}): "
                   f"{t_used:.1f} s for {f_used / 1e12:.2f} nominal NS TFLOP, extrapolated by nominal NS FLOPs "
                   f"to the whole owner step ({total / 1e12:.2f} TFLOP)"),
        "tflops_fp64": f_used / t_used / 1e12 if t_used else None,
    }


def cpu_baseline_tail(wl, hp, budget_s: float, cores: int):
    """The fp64 oracle's AdamW step on as many tail tensors as fit the budget,
    extrapolated to the whole tail by element count."""
    import numpy as np

    from oracle import muon_oracle as orc

    rng = np.random.default_rng(0)
    t_used, el_used, n = 0.0, 0, 0
    total = sum(s.numel for s in wl.specs)
    for s in wl.specs:
        if t_used > budget_s:
            break
        w = np.ones(s.numel)
        g = rng.standard_normal(s.numel) * s.grad_std
        z = np.zeros(s.numel)
        t0 = time.perf_counter()
        orc.adamw_step(w, g, z, z, 1, hp)
        t_used += time.perf_counter() - t0
        el_used += s.numel
        n += 1
    return {"value": t_used * total / el_used * 1e3, "unit": "ms", "cores": int(cores), "kind": "oracle",
            "sample": f"fp64 oracle AdamW step on {n} of {len(wl.specs)} tail tensors ({el_used} elements, "
                      f"{t_used:.1f} s), extrapolated by element count to the whole tail ({total} elements)"}


# HBM bytes per launch of the dominant kernel, from rocprofv3 counter runs
# (FETCH_SIZE x2 and WRITE_SIZE x1, the factors a plain device copy of known
# size reads back), keyed by workload, precision and phase, and valid only
# for the kernel sources they were taken with.
TRAFFIC = {
    # (workload, precision, phase): (sources sha256[:16], fetch bytes, write bytes)
    ("mixed-256-stress", "bf16", "update"): ("4de108779a05685d", 49695033376, 9145679872),
}
TRAFFIC_SOURCES = ("matrix_optimizer_owner_amd/csrc/ns_gemm.hip", "matrix_optimizer_owner_amd/csrc/plan.cpp",
                   "matrix_optimizer_owner_amd/csrc/layout.h")


def sources_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    root = os.path.dirname(os.path.abspath(__file__))
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(root, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, prec: str, phase: str):
    rec = TRAFFIC.get((workload, prec, phase))
    if rec is None or rec[0] != sources_digest():
        return None
    return rec[1] + rec[2]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--grad-pool-gb", type=float, default=48.0,
                    help="device memory for pre-generated per-step gradients")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--copy-probe-gib", type=float, default=0.0)
    ap.add_argument("--momentum-dtype", choices=("f32", "bf16"), default="f32",
                    help="storage type of the Muon momentum (the workloads state fp32)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the owner step on one GPU (the step has no cross-GPU work); "
              "--gpus above 1 is not supported.", file=sys.stderr)
        return 2
    if args.copy_probe_gib > 0:
        copy_probe(args.copy_probe_gib)
        return 0

    import torch

    from matrix_optimizer_owner_amd import binding as B
    from matrix_optimizer_owner_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    wl = W.config(args.config)
    hp = dict(wl.hparams, momentum_dtype=B.BF16 if args.momentum_dtype == "bf16" else B.F32)
    prec = "fp32" if int(hp.get("ns_precision", 0)) == 1 else "bf16"
    offs, pbytes = wl.layout()
    dt = {"bf16": B.BF16, "f32": B.F32}
    roles = {"auto": B.ROLE_AUTO, "muon": B.ROLE_MUON, "adamw": B.ROLE_ADAMW}
    entries = [B.TableEntry(o, s.rows, s.cols, dt[s.dtype], roles[s.role]) for o, s in zip(offs, wl.specs)]
    t0 = time.perf_counter()
    plan = B.OwnerPlan(entries, pbytes, B.make_hparams(**hp))
    plan_ms = (time.perf_counter() - t0) * 1e3
    dev = torch.device("cuda:0")
    u8 = torch.uint8
    params = torch.zeros(pbytes, dtype=u8, device=dev)
    state = torch.zeros(max(plan.state_bytes, 256), dtype=u8, device=dev)
    ws_bytes = max(plan.workspace_bytes, 256)
    ws = torch.zeros(ws_bytes, dtype=u8, device=dev)
    # a fresh seeded gradient per step (step t of the run draws the workload's
    # gradient stream t), generated before anything is timed
    n_grad = max(1, min(1 + args.warmup + args.steps, int(args.grad_pool_gb * 1e9 // pbytes)))
    grad_pool = [torch.zeros(pbytes, dtype=u8, device=dev) for _ in range(n_grad)]
    W.fill(wl, 1, params, grad_pool[0], params_too=True)
    for j in range(1, n_grad):
        W.fill(wl, j + 1, params, grad_pool[j], params_too=False)
    torch.cuda.synchronize()
    log(f"[bench] {wl.name}: {len(wl.muon_specs())} Muon matrices, params {pbytes / 1e9:.2f} GB, "
        f"state {plan.state_bytes / 1e9:.2f} GB, workspace {ws_bytes / 1e9:.2f} GB, "
        f"{n_grad} gradient buffers, plan {plan_ms:.1f} ms")

    hip = HipEvents()
    n_ev = plan.num_events()
    ev_sets = [hip.create(n_ev) for _ in range(args.steps)]
    stream = torch.cuda.current_stream().cuda_stream

    def one(step, events=(), resident=True):
        grads = grad_pool[(step - 1) % n_grad]
        plan.step(params.data_ptr(), grads.data_ptr(), state.data_ptr(), ws.data_ptr(), ws_bytes, step,
                  stream=stream, flags=B.STEP_DESCRIPTORS_RESIDENT if resident else 0, events=events)

    one(1, resident=False)  # uploads descriptors
    for i in range(args.warmup):
        one(2 + i)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        one(2 + args.warmup + k, events=ev_sets[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / args.steps

    # per-phase durations from the library's phase-boundary events
    steps_ns = int(hp.get("ns_steps", 5))
    ph = {"adamw": [], "momentum": [], "gram": [], "poly": [], "update": [], "final": [], "ns": []}
    step_ms = [hip.elapsed_ms(ev[0], ev[n_ev - 1]) for ev in ev_sets]
    for ev in ev_sets:
        ph["adamw"].append(hip.elapsed_ms(ev[0], ev[1]))
        ph["momentum"].append(hip.elapsed_ms(ev[1], ev[2]))
        if steps_ns:
            ph["ns"].append(hip.elapsed_ms(ev[2], ev[3 * steps_ns + 2]))
        for k in range(1, steps_ns + 1):
            ph["gram"].append(hip.elapsed_ms(ev[3 * k - 1], ev[3 * k]))
            ph["poly"].append(hip.elapsed_ms(ev[3 * k], ev[3 * k + 1]))
            # the last iteration's update kernel also writes the parameters
            ph["final" if k == steps_ns else "update"].append(hip.elapsed_ms(ev[3 * k + 1], ev[3 * k + 2]))
    for ev in ev_sets:
        hip.destroy(ev)

    def mean(v):
        return sum(v) / len(v) if v else 0.0

    specs = wl.muon_specs()
    gram_f = sum(2.0 * min(s.rows, s.cols) ** 2 * max(s.rows, s.cols) for s in specs)
    poly_f = sum(2.0 * min(s.rows, s.cols) ** 3 for s in specs)
    upd_f = gram_f
    per_launch = {"gram": gram_f, "poly": poly_f, "update": upd_f, "final": upd_f}
    tot = {k: sum(ph[k]) for k in per_launch}
    dom = max(tot, key=tot.get) if steps_ns and specs else None
    peak = PEAK_TFLOPS[prec]
    ns_ms = mean(ph["ns"])
    nominal = wl.nominal_ns_flops()
    muon_el = wl.muon_elements()
    tail_el = sum(s.numel for s in wl.specs if s not in specs and s.numel > 0)
    # AdamW moves W, g (storage type), m and v (fp32) in and W, m, v out
    tail_bytes = sum(s.numel * (3 * s.itemsize + 16) for s in wl.specs if s not in specs and s.numel > 0)
    # momentum pass: g read, momentum read and written, X0 written
    em = 2 if args.momentum_dtype == "bf16" else 4
    es_ns = 2 if prec == "bf16" else 4
    k1_bytes = sum(s.numel * (s.itemsize + 2 * em + es_ns) for s in specs)
    mom_ms = mean(ph["momentum"])
    adam_ms = mean(ph["adamw"])

    # executed NS FLOPs: the Gram and the polynomial compute upper tiles only
    # (256-tile edge when a phase has at least 512 of them, else 128, as the
    # planner chooses), on the padded shapes
    def executed_ns_flops():
        def pad(x):
            return (x + 255) // 256 * 256
        dims = [(pad(min(s.rows, s.cols)), pad(max(s.rows, s.cols))) for s in specs]
        def edge(count256):
            return 256 if count256 >= 512 else 128
        g_t = edge(sum((m // 256) * (m // 256 + 1) // 2 for m, _ in dims))
        u_t = edge(sum((m // 256) * (n // 256) for m, n in dims))
        gram = sum((m // g_t) * (m // g_t + 1) // 2 * g_t * g_t * 2.0 * n for m, n in dims)
        poly = sum((m // g_t) * (m // g_t + 1) // 2 * g_t * g_t * 2.0 * m for m, n in dims)
        upd = sum(2.0 * m * m * n for m, n in dims)
        return steps_ns * (gram + poly + upd)

    # device-copy ceiling of this GPU, measured live (1 GiB read + 1 GiB written)
    cbuf = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    csrc, cdst = cbuf[: 1 << 30], cbuf[1 << 30:]
    for _ in range(2):
        cdst.copy_(csrc)
    torch.cuda.synchronize()
    c0 = time.perf_counter()
    for _ in range(5):
        cdst.copy_(csrc)
    torch.cuda.synchronize()
    copy_gbs = 2.0 * (1 << 30) * 5 / (time.perf_counter() - c0) / 1e9
    # streaming rates with the library's probe (16-byte accesses over 1 GiB):
    # read only, write only, copy (the read/write mix of the elementwise phases)
    hbm = {}
    hsink = torch.empty(8192, dtype=torch.float32, device=dev)
    for name, mode, moved in (("read", 0, 1), ("write", 1, 1), ("copy", 2, 2)):
        B.probe_hbm(cdst.data_ptr(), csrc.data_ptr(), 1 << 30, mode, hsink.data_ptr(), stream)  # warm-up
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            B.probe_hbm(cdst.data_ptr(), csrc.data_ptr(), 1 << 30, mode, hsink.data_ptr(), stream)
        e1.record()
        torch.cuda.synchronize()
        hbm[name + "_gbs"] = round(moved * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del cbuf, csrc, cdst, hsink

    # bf16 MFMA rate this GPU sustains, measured live on register-only MFMA
    # loops (one block of 4 waves per CU, about 60 ms each, long enough for the
    # clock to settle): the clock under load depends on the operand data, so
    # Gaussian bf16 (the contractions' kind of data) and zeros.  The operands
    # stay in registers (16 fragments per lane), so fewer operand bits toggle
    # than in a contraction streaming fresh fragments: an upper bound on what
    # a contraction can sustain on such data.
    mfma_ceiling = None
    if prec == "bf16":
        ops = torch.randn(1 << 22, device=dev, dtype=torch.float32).to(torch.bfloat16)
        sink = torch.empty(256 * 4, dtype=torch.float32, device=dev)
        mfma_ceiling = {}
        for name, buf in (("gaussian_bf16", ops), ("zeros", torch.zeros_like(ops))):
            B.probe_mfma_bf16(buf.data_ptr(), buf.numel() * 2, 256, 2000, sink.data_ptr(), stream)  # warm-up
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fl = B.probe_mfma_bf16(buf.data_ptr(), buf.numel() * 2, 256, 100000, sink.data_ptr(), stream)
            e1.record()
            torch.cuda.synchronize()
            mfma_ceiling[name + "_tflops"] = round(fl / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del ops, sink

    roofline = None
    if not specs and adam_ms:
        # tail-only buffer: the AdamW kernel is the step (28 B per fp32 element)
        ach = tail_bytes / (adam_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None, "kernel": "k_adamw",
                    "avg_launch_ms": round(adam_ms, 4), "algorithmic_bytes_per_launch": tail_bytes}
    if dom:
        avg = mean(ph[dom])
        ach = per_launch[dom] / (avg * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                    "frac": round(ach / peak, 4), "traffic": measured_traffic(wl.name, prec, dom),
                    "measured_mfma_ceiling": mfma_ceiling,
                    "frac_of_measured_ceiling": (round(ach / mfma_ceiling["gaussian_bf16_tflops"], 4)
                                                 if mfma_ceiling else None),
                    "kernel": f"k_ns_gemm ({dom} phase)", "avg_launch_ms": round(avg, 4),
                    "algorithmic_flop_per_launch": per_launch[dom]}

    out = {
        "metric": METRIC,
        "value": round(ms, 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": prec if specs else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "muon_matrices": len(specs), "muon_elements": muon_el,
                   "tail_tensors": sum(1 for s in wl.specs if s not in specs and s.numel > 0),
                   "tail_elements": tail_el, "ns_steps": steps_ns, "momentum_dtype": args.momentum_dtype,
                   "fresh_gradient_buffers": n_grad, "parallelism": "single GPU owner"},
        "step_ms_median": round(sorted(step_ms)[len(step_ms) // 2], 4),
        "step_ms_p90": round(sorted(step_ms)[min(len(step_ms) - 1, int(0.9 * len(step_ms)))], 4),
        "step_ms_all": [round(x, 4) for x in step_ms],
        "matrices_per_s": round(len(specs) / (ms * 1e-3), 2),
        "ns_tflops_nominal": round(nominal / (ns_ms * 1e-3) / 1e12, 2) if ns_ms else None,
        "ns_frac_peak": round(nominal / (ns_ms * 1e-3) / 1e12 / peak, 4) if ns_ms else None,
        "ns_meets_60pct_target": (nominal / (ns_ms * 1e-3) / 1e12 / peak >= 0.60) if ns_ms else None,
        "ns_tflops_executed": round(executed_ns_flops() / (ns_ms * 1e-3) / 1e12, 2) if ns_ms else None,
        "step_tflops_nominal": round(nominal / (ms * 1e-3) / 1e12, 2),
        "phases_ms": {"adamw": round(adam_ms, 4), "momentum_norm": round(mom_ms, 4), "ns_total": round(ns_ms, 4),
                      "gram_avg": round(mean(ph["gram"]), 4), "poly_avg": round(mean(ph["poly"]), 4),
                      "update_avg": round(mean(ph["update"]), 4), "final_update": round(mean(ph["final"]), 4)},
        "elementwise": {"momentum_gbs": round(k1_bytes / (mom_ms * 1e-3) / 1e9, 1) if mom_ms else None,
                        "momentum_frac_hbm": round(k1_bytes / (mom_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if mom_ms else None,
                        "momentum_bytes_per_elem": round(k1_bytes / muon_el, 3) if muon_el else None,
                        "copy_ceiling_gbs": round(copy_gbs, 1),
                        "hbm_stream_probe": hbm,
                        "momentum_frac_copy_ceiling": round(k1_bytes / (mom_ms * 1e-3) / 1e9 / copy_gbs, 4) if mom_ms else None,
                        "adamw_gbs": round(tail_bytes / (adam_ms * 1e-3) / 1e9, 1) if adam_ms and tail_el else None,
                        # the target is 70% of the published 8 TB/s; the copy-ceiling fraction above
                        # says how close the pass is to what a read+write stream reaches here, not that
                        # the target is met
                        "target_frac_hbm": 0.70,
                        "momentum_meets_target": (k1_bytes / (mom_ms * 1e-3) / 1e9 / PEAK_HBM_GBS >= 0.70)
                        if mom_ms else None},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    log(f"[bench] {ms:.3f} ms/step; NS {out['ns_tflops_nominal']} TFLOP/s nominal")
    if not args.no_cpu_baseline:
        log(f"[bench] timing the fp64 oracle on host cores (budget {args.cpu_budget_s:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
