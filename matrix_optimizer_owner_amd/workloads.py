"""Seeded synthetic owner buffers: shapes, dtypes, packing and values.

This module holds no optimizer arithmetic.  It only says which tensors an
owner holds (the shapes of GPT-2-small, a Llama-3-8B owner share, a
Llama-3-70B owner share, a mixed-shape stress set, and small ragged cases),
how they are packed into one flat byte buffer, and how their values are
drawn.  Both the HIP path's tests/benchmark and the oracle receive the same
stored values from here (the oracle reads them back from the device buffers).

Value recipe: parameters ~ N(0, 0.02) unless a tensor is a LayerNorm gain
(ones) or a bias (zeros); gradients ~ N(0, grad_std).  Each tensor and step
draws from its own stream, keyed by (workload seed, step, entry index,
kind), so any single tensor can be regenerated alone.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np

ALIGN = 256
KIND_PARAM, KIND_GRAD = 0, 1


@dataclass(frozen=True)
class TensorSpec:
    name: str
    rows: int
    cols: int
    dtype: str = "bf16"        # "bf16" or "f32", parameter and gradient
    init: str = "normal"       # "normal" (N(0, param_std)), "ones", "zeros"
    param_std: float = 0.02
    grad_std: float = 1e-3
    role: str = "auto"         # "auto", "muon", "adamw"

    @property
    def numel(self) -> int:
        return self.rows * self.cols

    @property
    def itemsize(self) -> int:
        return 2 if self.dtype == "bf16" else 4


@dataclass
class Workload:
    name: str
    specs: List[TensorSpec]
    seed: int
    steps: int = 1
    hparams: Dict[str, float] = field(default_factory=dict)
    note: str = ""

    def layout(self) -> Tuple[List[int], int]:
        """Byte offsets of every tensor in the flat buffer (256-byte aligned,
        table order) and the buffer size."""
        offs, off = [], 0
        for s in self.specs:
            offs.append(off)
            off = (off + s.numel * s.itemsize + ALIGN - 1) // ALIGN * ALIGN
        return offs, max(off, ALIGN)

    def muon_specs(self) -> List[TensorSpec]:
        return [s for s in self.specs if (s.role == "muon") or (s.role == "auto" and s.rows > 1 and s.cols > 1)]

    def muon_elements(self) -> int:
        return sum(s.numel for s in self.muon_specs())

    def nominal_ns_flops(self) -> float:
        """Nominal Newton-Schulz FLOPs of one step: (4 m^2 n + 2 m^3) per
        iteration per matrix with m = min dim, n = max dim."""
        steps = int(self.hparams.get("ns_steps", 5))
        tot = 0.0
        for s in self.muon_specs():
            m, n = min(s.rows, s.cols), max(s.rows, s.cols)
            tot += steps * (4.0 * m * m * n + 2.0 * m ** 3)
        return tot


# ---------------------------------------------------------------------------
# The five workloads
# ---------------------------------------------------------------------------

MUON_DEFAULTS = dict(lr=0.02, weight_decay=0.01, momentum=0.95, nesterov=1, ns_steps=5,
                     ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315, ns_eps=1e-7, lr_scale_mode=0,
                     adam_lr=0.02, adam_beta1=0.9, adam_beta2=0.95, adam_eps=1e-8, adam_weight_decay=0.01)


def single_fp32() -> Workload:
    """One 256x512 fp32 weight, gradient ~ N(0, 1), fp32 Newton-Schulz."""
    hp = dict(MUON_DEFAULTS, ns_precision=1)
    return Workload("single-256x512-fp32", [TensorSpec("w", 256, 512, "f32", grad_std=1.0)], seed=0,
                    hparams=hp)


def gpt2_small() -> Workload:
    """GPT-2-small owner buffer: 12 layers of c_attn 768x2304, attn c_proj
    768x768, c_fc 768x3072, mlp c_proj 3072x768 (bf16, HF Conv1D
    orientation), plus the fp32 AdamW tail: LayerNorm gains/biases and
    biases (98 tensors, 121,344 elements)."""
    sp: List[TensorSpec] = []
    d, f = 768, 3072
    for l in range(12):
        p = f"h{l}."
        sp += [
            TensorSpec(p + "ln_1.weight", 1, d, "f32", "ones"),
            TensorSpec(p + "ln_1.bias", 1, d, "f32", "zeros"),
            TensorSpec(p + "attn.c_attn.weight", d, 3 * d),
            TensorSpec(p + "attn.c_attn.bias", 1, 3 * d, "f32", "zeros"),
            TensorSpec(p + "attn.c_proj.weight", d, d),
            TensorSpec(p + "attn.c_proj.bias", 1, d, "f32", "zeros"),
            TensorSpec(p + "ln_2.weight", 1, d, "f32", "ones"),
            TensorSpec(p + "ln_2.bias", 1, d, "f32", "zeros"),
            TensorSpec(p + "mlp.c_fc.weight", d, f),
            TensorSpec(p + "mlp.c_fc.bias", 1, f, "f32", "zeros"),
            TensorSpec(p + "mlp.c_proj.weight", f, d),
            TensorSpec(p + "mlp.c_proj.bias", 1, d, "f32", "zeros"),
        ]
    sp += [TensorSpec("ln_f.weight", 1, d, "f32", "ones"), TensorSpec("ln_f.bias", 1, d, "f32", "zeros")]
    return Workload("gpt2-small-owner", sp, seed=1, hparams=dict(MUON_DEFAULTS, ns_precision=0))


def llama3_8b_share() -> Workload:
    """One owner's 1/8 share of Llama-3-8B: 4 layers of q,o 4096x4096,
    k,v 1024x4096, gate,up 14336x4096, down 4096x14336; grads ~ N(0, 1e-4);
    10 consecutive steps."""
    sp = []
    for l in range(4):
        p = f"l{l}."
        sp += [
            TensorSpec(p + "q", 4096, 4096, grad_std=1e-4), TensorSpec(p + "k", 1024, 4096, grad_std=1e-4),
            TensorSpec(p + "v", 1024, 4096, grad_std=1e-4), TensorSpec(p + "o", 4096, 4096, grad_std=1e-4),
            TensorSpec(p + "gate", 14336, 4096, grad_std=1e-4), TensorSpec(p + "up", 14336, 4096, grad_std=1e-4),
            TensorSpec(p + "down", 4096, 14336, grad_std=1e-4),
        ]
    return Workload("llama3-8b-owner-share-4L", sp, seed=2, steps=10, hparams=dict(MUON_DEFAULTS, ns_precision=0))


def mixed_stress(count: int = 256) -> Workload:
    """Mixed shapes: min dim uniform in {512,1024,2048,4096}, aspect in
    {1,2,4,8}, tall or wide by a fair coin, grads N(0,1) scaled per matrix
    by 10^U(-5,-1).  Drawn with numpy default_rng(3)."""
    rng = np.random.default_rng(3)
    sp = []
    for i in range(count):
        m = int(rng.choice([512, 1024, 2048, 4096]))
        r = int(rng.choice([1, 2, 4, 8]))
        tall = bool(rng.random() < 0.5)
        scale = float(10.0 ** rng.uniform(-5.0, -1.0))
        rows, cols = (m * r, m) if tall else (m, m * r)
        sp.append(TensorSpec(f"mat{i}", rows, cols, grad_std=scale))
    return Workload("mixed-256-stress", sp, seed=3, hparams=dict(MUON_DEFAULTS, ns_precision=0))


def llama3_70b_share() -> Workload:
    """Large-matrix owner share of Llama-3-70B: 2 layers of q,o 8192x8192,
    k,v 1024x8192, gate,up 28672x8192, down 8192x28672; grads ~ N(0, 1e-4)."""
    sp = []
    for l in range(2):
        p = f"l{l}."
        sp += [
            TensorSpec(p + "q", 8192, 8192, grad_std=1e-4), TensorSpec(p + "k", 1024, 8192, grad_std=1e-4),
            TensorSpec(p + "v", 1024, 8192, grad_std=1e-4), TensorSpec(p + "o", 8192, 8192, grad_std=1e-4),
            TensorSpec(p + "gate", 28672, 8192, grad_std=1e-4), TensorSpec(p + "up", 28672, 8192, grad_std=1e-4),
            TensorSpec(p + "down", 8192, 28672, grad_std=1e-4),
        ]
    return Workload("llama3-70b-owner-share-2L", sp, seed=4, hparams=dict(MUON_DEFAULTS, ns_precision=0))


def adamw_tail_probe() -> Workload:
    """Tail-only owner buffer for measuring the AdamW kernel where HBM bounds
    it: 64 fp32 vectors of 4 Mi elements (268 M elements, 7.5 GB moved per
    step).  Not one of the five workloads; the GPT-2 tail (121,344
    elements) is too small for its time to say anything about bandwidth."""
    sp = [TensorSpec(f"tail{i}", 1, 4 << 20, "f32", "zeros" if i % 2 else "ones", grad_std=1e-3) for i in range(64)]
    return Workload("adamw-tail-64x4Mi-fp32", sp, seed=7, hparams=dict(MUON_DEFAULTS, ns_precision=0))


WORKLOADS = [single_fp32, gpt2_small, llama3_8b_share, mixed_stress, llama3_70b_share, adamw_tail_probe]


def config(i: int) -> Workload:
    return WORKLOADS[i]()


def small_ragged(seed: int = 5, precision: int = 0) -> Workload:
    """Small mixed table for parity: ragged shapes (not multiples of any
    tile), tall and wide, a square, an fp32 Muon matrix, a 1xN and an Nx1
    tail, an empty shard, and a matrix spanning several 128-tiles."""
    sp = [
        TensorSpec("wide_ragged", 100, 300, grad_std=1e-3),
        TensorSpec("tall_ragged", 520, 130, grad_std=1e-2),
        TensorSpec("square", 256, 256, grad_std=1.0),
        TensorSpec("fp32_mat", 72, 200, "f32", grad_std=1e-3),
        TensorSpec("bias", 1, 333, "f32", "zeros"),
        TensorSpec("column", 77, 1, "f32", "ones"),
        TensorSpec("empty", 0, 64),
        TensorSpec("multi_tile", 384, 700, grad_std=1e-4),
        TensorSpec("odd_cols", 33, 45, grad_std=1e-3),
        TensorSpec("bf16_tail", 1, 1000, "bf16", grad_std=1e-3),
    ]
    return Workload(f"small-ragged-p{precision}", sp, seed=seed, hparams=dict(MUON_DEFAULTS, ns_precision=precision))


# ---------------------------------------------------------------------------
# Values
# ---------------------------------------------------------------------------

def stream_seed(seed: int, step: int, index: int, kind: int) -> int:
    """63-bit seed of one tensor's value stream."""
    st = np.random.SeedSequence([seed, step, index, kind]).generate_state(2, np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def fill(workload: Workload, step: int, params, grads, which: Sequence[int] = None,
         params_too: bool = True) -> None:
    """Write seeded values into flat uint8 torch buffers (CPU or CUDA).

    Parameters are drawn with step 0 (initial weights); gradients with the
    given 1-based step.  ``which`` limits the fill to some entries.
    """
    import torch

    offs, _ = workload.layout()
    dev = params.device
    gen = torch.Generator(device=dev)
    idxs = range(len(workload.specs)) if which is None else which
    for i in idxs:
        s = workload.specs[i]
        if s.numel == 0:
            continue
        tdt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
        nbytes = s.numel * s.itemsize
        if params_too:
            pv = params[offs[i]:offs[i] + nbytes].view(tdt)
            if s.init == "ones":
                pv.fill_(1.0)
            elif s.init == "zeros":
                pv.zero_()
            else:
                gen.manual_seed(stream_seed(workload.seed, 0, i, KIND_PARAM))
                pv.copy_(torch.randn(s.numel, generator=gen, device=dev, dtype=torch.float32) * s.param_std)
        gv = grads[offs[i]:offs[i] + nbytes].view(tdt)
        gen.manual_seed(stream_seed(workload.seed, step, i, KIND_GRAD))
        gv.copy_(torch.randn(s.numel, generator=gen, device=dev, dtype=torch.float32) * s.grad_std)
