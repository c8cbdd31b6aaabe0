"""GPU checks of what the step leaves alone.

* Guard bands: every caller buffer gets 64 KiB of canary bytes before and
  after it, and the plan leaves a guard gap after every state and workspace
  region it lays out (hparams.guard_bytes, listed by mfsdp_plan_regions).
  The canary is 0xFF in every byte, a NaN in both bf16 and fp32, and it
  also fills the workspace regions themselves, so a kernel that read a
  workspace byte before writing it would poison its result.  After two
  steps every byte outside the regions, the tensors and the O export must
  still be the canary, the gradients untouched, and every result bitwise
  equal to a run on zero-filled buffers without guards.
* Non-finite gradients propagate and are not masked: a NaN or an Inf in one
  Muon matrix's gradient makes that matrix's whole O and parameter update
  non-finite (the Frobenius norm and the Newton-Schulz products mix every
  element) and its momentum non-finite at that element only; an Inf in an
  AdamW tensor makes only that element non-finite.  Every other entry is
  bitwise equal to a clean run.
"""

import numpy as np
import pytest

from matrix_optimizer_owner_amd import binding as B
from matrix_optimizer_owner_amd import workloads as W
from tests.harness import DT, ROLE, DeviceRun, say
from tests.test_random_shapes_gpu import random_table

pytestmark = pytest.mark.gpu

MARGIN = 64 << 10
CANARY = 0xFF
GUARD = 4096


def _reference(wl, steps, hp=None):
    """Params, per-entry state and O of a plain run (zero-filled buffers, no
    guards), as host arrays, after each step."""
    run = DeviceRun(wl, hp)
    out = []
    try:
        for t in range(1, steps + 1):
            run.fill(t, params_too=(t == 1))
            run.run(t)
            h = run.host()
            out.append({"params": h["params"], "state": {}, "o": {}})
            for i, inf in enumerate(run.info):
                s = wl.specs[i]
                if inf.role == B.ROLE_MUON:
                    mb = 4 * s.numel
                    out[-1]["state"][(i, 1)] = h["state"][inf.state_offset:inf.state_offset + mb].copy()
                    out[-1]["o"][i] = h["ns_out"][inf.ns_out_offset:inf.ns_out_offset + s.numel].copy()
                elif inf.role == B.ROLE_ADAMW:
                    out[-1]["state"][(i, 1)] = h["state"][inf.state_offset:inf.state_offset + 4 * s.numel].copy()
                    out[-1]["state"][(i, 2)] = h["state"][inf.state_offset2:inf.state_offset2 + 4 * s.numel].copy()
    finally:
        run.free()
    return out


def _mask(nbytes, spans):
    """Boolean mask of a buffer with MARGIN on both sides: True outside the
    given (offset, bytes) spans (offsets relative to the buffer start)."""
    m = np.ones(nbytes + 2 * MARGIN, dtype=bool)
    for off, n in spans:
        m[MARGIN + off:MARGIN + off + n] = False
    return m


@pytest.mark.parametrize("which", ["gpt2-small-owner", "random-table"])
def test_guard_bands(which):
    import torch

    wl = W.config(1) if which == "gpt2-small-owner" else random_table(21, 0)
    steps = 2
    ref = _reference(wl, steps)
    offs, pbytes = wl.layout()
    entries = [B.TableEntry(o, s.rows, s.cols, DT[s.dtype], ROLE[s.role]) for o, s in zip(offs, wl.specs)]
    plan = B.OwnerPlan(entries, pbytes, B.make_hparams(**dict(wl.hparams, guard_bytes=GUARD)))
    regions = plan.regions()
    info = [plan.entry_info(i) for i in range(len(entries))]
    dev = torch.device("cuda")

    def alloc(nbytes):
        base = torch.full((nbytes + 2 * MARGIN,), CANARY, dtype=torch.uint8, device=dev)
        return base, base[MARGIN:MARGIN + nbytes]

    sbytes, wbytes = max(plan.state_bytes, 256), max(plan.workspace_bytes, 256)
    obytes = 4 * max(plan.ns_out_elems, 4)
    p_base, params = alloc(pbytes)
    g_base, grads = alloc(pbytes)
    s_base, state = alloc(sbytes)
    w_base, ws = alloc(wbytes)
    o_base, o_u8 = alloc(obytes)
    for r in regions:
        if r.buffer == B.BUFFER_STATE:
            state[r.offset:r.offset + r.bytes].zero_()  # the state starts at zero; the gaps stay canary
    # which bytes the step may touch
    ent_spans = [(offs[i], s.numel * s.itemsize) for i, s in enumerate(wl.specs) if s.numel > 0]
    st_spans = [(r.offset, r.bytes) for r in regions if r.buffer == B.BUFFER_STATE]
    ws_spans = [(r.offset, r.bytes) for r in regions if r.buffer == B.BUFFER_WORKSPACE]
    o_spans = [(4 * inf.ns_out_offset, 4 * wl.specs[i].numel) for i, inf in enumerate(info) if inf.role == B.ROLE_MUON]
    say(f"[guard {which}] {len(regions)} regions, guard {GUARD} B, margins {MARGIN} B; "
        f"state {sbytes} B, workspace {wbytes} B")
    stream = torch.cuda.current_stream().cuda_stream
    try:
        for t in range(1, steps + 1):
            W.fill(wl, t, params, grads, params_too=(t == 1))
            torch.cuda.synchronize()
            g_before = g_base.cpu().numpy()
            p_before = p_base.cpu().numpy()
            plan.step(params.data_ptr(), grads.data_ptr(), state.data_ptr(), ws.data_ptr(), wbytes, t, stream=stream,
                      ns_out=o_u8.data_ptr(), flags=B.STEP_DESCRIPTORS_RESIDENT if t > 1 else 0)
            torch.cuda.synchronize()
            g_after, p_after = g_base.cpu().numpy(), p_base.cpu().numpy()
            s_after, w_after, o_after = s_base.cpu().numpy(), w_base.cpu().numpy(), o_base.cpu().numpy()
            assert np.array_equal(g_after, g_before), "gradients changed"
            mp = _mask(pbytes, ent_spans)
            assert np.array_equal(p_after[mp], p_before[mp]), "bytes between or around the tensors changed"
            for name, buf, n, spans in (("state", s_after, sbytes, st_spans), ("workspace", w_after, wbytes, ws_spans),
                                        ("ns_out", o_after, obytes, o_spans)):
                m = _mask(n, spans)
                bad = np.flatnonzero(buf[m] != CANARY)
                say(f"  [guard {which} t={t}] {name}: {int(m.sum())} canary bytes, {bad.size} changed")
                assert bad.size == 0, f"{name}: {bad.size} canary bytes overwritten"
            # results equal the plain run's, bit for bit
            r = ref[t - 1]
            for off, n in ent_spans:
                assert np.array_equal(p_after[MARGIN + off:MARGIN + off + n], r["params"][off:off + n]), \
                    f"params at byte {off} differ"
            o32 = o_after[MARGIN:MARGIN + obytes].view(np.float32)
            for i, inf in enumerate(info):
                s = wl.specs[i]
                if inf.role == B.ROLE_MUON:
                    got = s_after[MARGIN + inf.state_offset:MARGIN + inf.state_offset + 4 * s.numel]
                    assert np.array_equal(got, r["state"][(i, 1)]), f"momentum of {s.name}"
                    o = o32[inf.ns_out_offset:inf.ns_out_offset + s.numel]
                    assert np.array_equal(o.view(np.uint32), r["o"][i].view(np.uint32)), f"O of {s.name}"
                elif inf.role == B.ROLE_ADAMW:
                    for k, off in ((1, inf.state_offset), (2, inf.state_offset2)):
                        got = s_after[MARGIN + off:MARGIN + off + 4 * s.numel]
                        assert np.array_equal(got, r["state"][(i, k)]), f"AdamW moment {k} of {s.name}"
    finally:
        del p_base, g_base, s_base, w_base, o_base
        torch.cuda.empty_cache()


@pytest.mark.parametrize("tile", [0, 256])
def test_nonfinite_gradients_propagate_and_stay_local(tile):
    import torch

    wl = W.small_ragged(precision=0)
    names = [s.name for s in wl.specs]
    nan_mat, inf_mat, inf_tail = names.index("multi_tile"), names.index("tall_ragged"), names.index("bias")
    hp = {"ns_tile": tile}
    clean = DeviceRun(wl, hp)
    bad = DeviceRun(wl, hp)
    try:
        for run in (clean, bad):
            run.fill(1, params_too=True)
        spots = ((nan_mat, (5, 7), float("nan")), (inf_mat, (400, 3), float("inf")), (inf_tail, (0, 3), float("inf")))
        for i, (r, c), v in spots:
            s = wl.specs[i]
            el = bad.offs[i] + (r * s.cols + c) * s.itemsize
            view = bad.grads[el:el + s.itemsize].view(torch.bfloat16 if s.dtype == "bf16" else torch.float32)
            view.fill_(v)
        for run in (clean, bad):
            run.run(1)
        say(f"[nonfinite tile={tile}] NaN in {names[nan_mat]}, Inf in {names[inf_mat]} and {names[inf_tail]}")
        poisoned = {nan_mat, inf_mat, inf_tail}
        for i, s in enumerate(wl.specs):
            inf = clean.info[i]
            if inf.role == -1:
                continue
            whats = ["param", "state"] + (["o"] if inf.role == B.ROLE_MUON else ["state2"])
            got = {w: bad.dev_entry(i, w) for w in whats}
            want = {w: clean.dev_entry(i, w) for w in whats}
            if i not in poisoned:
                for w in whats:
                    assert np.array_equal(got[w], want[w], equal_nan=True), f"{s.name} {w} changed"
                continue
            r, c = next((rc for k, rc, _ in spots if k == i))
            if inf.role == B.ROLE_MUON:
                # the whole update is non-finite; the momentum only at the spot
                assert not np.isfinite(got["o"]).any(), f"{s.name}: finite O left"
                assert not np.isfinite(got["param"]).any(), f"{s.name}: finite W left"
                m_ok = np.ones(got["state"].shape, dtype=bool)
                m_ok[r, c] = False
                assert not np.isfinite(got["state"][r, c])
                assert np.array_equal(got["state"][m_ok], want["state"][m_ok])
            else:
                m_ok = np.ones(got["param"].shape, dtype=bool)
                m_ok[r, c] = False
                assert np.isnan(got["param"][r, c]) and np.isinf(got["state"][r, c]) and np.isinf(got["state2"][r, c])
                for w in whats:
                    assert np.array_equal(got[w][m_ok], want[w][m_ok]), f"{s.name} {w} changed off the spot"
            say(f"  {s.name}: non-finite where expected, bitwise equal elsewhere")
    finally:
        clean.free()
        bad.free()
