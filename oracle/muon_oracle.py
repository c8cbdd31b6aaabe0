"""Plain fp64 CPU oracle for the owner-local Muon + AdamW optimizer step.

TEST INFRASTRUCTURE ONLY.  This module is the slow, obviously-correct
statement of what the owner step computes.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it.  The product path
(the HIP library and its Python binding) never imports, calls or links
anything here, and this module imports nothing from the product path.

Source of the method: "MatrixFSDP: Communication-Free Matrix Optimizers
Under ZeRO-3 Parameter Sharding" (arXiv 2607.05895).  Its Abstract states
that Muon orthogonalises momentum-smoothed matrix updates with
Newton-Schulz, that each 2D weight is handled whole on its owner, that
the remaining (non-matrix) tensors are optimised with AdamW, and that the
result must equal full-matrix Muon computed on the gathered matrix
(Abstract; §1).  The pages give no formulas, so every
numeric choice below is a plain reading, listed in the design notes:

* momentum: SGD-Nesterov form, m <- beta*m + g, u <- g + beta*m
  (Muon of Jordan et al. 2024, the Muon reference cited in §1);
* Frobenius normalisation of the Newton-Schulz input with eps added to
  the norm;
* quintic Newton-Schulz with coefficients (a, b, c) applied to the wide
  orientation (fewer rows than columns);
* learning-rate shape scale sqrt(max(1, rows/cols)) (mode 0) or
  0.2*sqrt(max(rows, cols)) (mode 1, Liu et al. 2025, also cited in §1);
* decoupled weight decay scaled by the learning rate;
* AdamW in the bias-corrected, decoupled-decay form.

Arithmetic is fp64 throughout; hyper-parameters are the float32 values the
library receives, widened to fp64.  Matrix products use numpy's ``@``
(BLAS DGEMM) as a library primitive; nothing is blocked, fused or reordered.

Parity pins (tests/test_oracle_pins.py): Newton-Schulz against the SVD
closed form U p^5(S) V^T (the matrix form and the vector-applied form),
unchanged singular vectors, the output-band invariant, transpose symmetry (direct large-Gram evaluation), exact special
cases (zero, rank-1, [I 0]), scale invariance, momentum closed forms, AdamW
step-1 and constant-gradient closed forms, and bf16 rounding against an
exhaustive enumeration.  The learning-rate shape-scale convention and the
AdamW lr/decay values are definitions, not derivations: "parity unpinned"
by the pages for those choices (the arithmetic that applies them is pinned).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------------------
# Hyper-parameters
# ---------------------------------------------------------------------------

def f32(x: float) -> float:
    """The float32 value a float hyper-parameter has once it crosses the
    C ABI, widened back to a Python float (fp64)."""
    return float(np.float32(x))


@dataclass(frozen=True)
class Hparams:
    """Muon + AdamW hyper-parameters, held as fp64 copies of float32 values."""

    lr: float = f32(0.02)
    weight_decay: float = f32(0.01)
    momentum: float = f32(0.95)
    nesterov: bool = True
    ns_steps: int = 5
    ns_a: float = f32(3.4445)
    ns_b: float = f32(-4.7750)
    ns_c: float = f32(2.0315)
    ns_eps: float = f32(1e-7)
    lr_scale_mode: int = 0
    adam_lr: float = f32(0.02)
    adam_beta1: float = f32(0.9)
    adam_beta2: float = f32(0.95)
    adam_eps: float = f32(1e-8)
    adam_weight_decay: float = f32(0.01)


# ---------------------------------------------------------------------------
# Newton-Schulz orthogonalisation (Abstract: Muon's update is the
# momentum-smoothed matrix made near-orthogonal by Newton-Schulz)
# ---------------------------------------------------------------------------

def newton_schulz(x: np.ndarray, steps: int, a: float, b: float, c: float) -> np.ndarray:
    """Quintic Newton-Schulz on a 2D array, returned in the input's shape.

    The iteration runs on the wide orientation (rows <= cols), where the
    Gram matrix X X^T is the smaller one; a tall input is transposed first
    and the result transposed back.  Each iteration:
        A = X X^T,   B = b A + c A A,   X <- a X + B X.
    """
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("newton_schulz expects a 2D array")
    tall = x.shape[0] > x.shape[1]
    xw = x.T.copy() if tall else x.copy()
    for _ in range(steps):
        gram = xw @ xw.T
        poly = b * gram + c * (gram @ gram)
        xw = a * xw + poly @ xw
    return xw.T.copy() if tall else xw


def newton_schulz_apply(x: np.ndarray, v: np.ndarray, steps: int, a: float, b: float, c: float) -> np.ndarray:
    """NS_steps(X) @ V for a block of vectors V, without forming any matrix
    product of X with itself: the same iteration, applied to vectors.

    With X_0 = X (wide orientation) and X_k = a X_{k-1} + B_{k-1} X_{k-1},
    B = b A + c A A, A = X_{k-1} X_{k-1}^T:
        X_k y   = a z + b A z + c A (A z),   z = X_{k-1} y
        X_k^T w = X_{k-1}^T (a w + b A w + c A (A w))   (B is symmetric)
    and A z = X_{k-1} (X_{k-1}^T z).  The cost is about 5^k products of X_0
    with a vector block, so this is for few steps on large matrices.  A tall
    X is handled through its transpose, as in newton_schulz.
    """
    x = np.asarray(x, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    tall = x.shape[0] > x.shape[1]
    xw = x.T if tall else x

    def fwd(k, y):  # X_k y  (wide: m x n times n-vectors)
        if k == 0:
            return xw @ y
        z = fwd(k - 1, y)
        return _poly(k - 1, z)

    def bwd(k, w):  # X_k^T w
        if k == 0:
            return xw.T @ w
        return bwd(k - 1, _poly(k - 1, w))

    def _gram(k, z):  # A_k z = X_k (X_k^T z)
        return fwd(k, bwd(k, z))

    def _poly(k, z):  # (a I + b A_k + c A_k A_k) z
        az = _gram(k, z)
        return a * z + b * az + c * _gram(k, az)

    if tall:  # X = X_w^T and NS(X) = NS(X_w)^T, so NS(X) V = NS(X_w)^T V
        return bwd(steps, v)
    return fwd(steps, v)


def frobenius_normalise(u: np.ndarray, eps: float) -> np.ndarray:
    """X = U / (||U||_F + eps): the Newton-Schulz input."""
    u = np.asarray(u, dtype=np.float64)
    return u / (math.sqrt(float(np.sum(u * u))) + eps)


def lr_shape_scale(rows: int, cols: int, mode: int) -> float:
    """Per-matrix learning-rate multiplier.

    mode 0: sqrt(max(1, rows/cols)) (Muon, Jordan et al. 2024);
    mode 1: 0.2*sqrt(max(rows, cols)) (Liu et al. 2025).
    """
    if mode == 0:
        return math.sqrt(max(1.0, rows / cols))
    if mode == 1:
        return 0.2 * math.sqrt(max(rows, cols))
    raise ValueError(f"unknown lr_scale_mode {mode}")


# ---------------------------------------------------------------------------
# Muon step on one whole matrix (Abstract: the owner holds the whole matrix,
# so the update equals full-matrix Muon)
# ---------------------------------------------------------------------------

def momentum_step(m, g, hp: Hparams):
    """Momentum smoothing: m <- beta m + g; the Newton-Schulz input is
    u = g + beta m (Nesterov) or u = m.  Returns (m_new, u)."""
    m = np.asarray(m, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = hp.momentum
    m_new = beta * m + g
    u = g + beta * m_new if hp.nesterov else m_new
    return m_new, u


def apply_update(w, o, rows: int, cols: int, hp: Hparams):
    """W <- W (1 - lr wd) - lr * scale * O (decoupled weight decay)."""
    w = np.asarray(w, dtype=np.float64)
    scale = lr_shape_scale(rows, cols, hp.lr_scale_mode)
    return w * (1.0 - hp.lr * hp.weight_decay) - hp.lr * scale * np.asarray(o, dtype=np.float64)


def muon_matrix_step(w, g, m, hp: Hparams):
    """One Muon step for one whole matrix, all fp64.

    Returns (w_new, m_new, o) where o is the orthogonalised update in the
    matrix's own orientation.
    """
    w = np.asarray(w, dtype=np.float64)
    rows, cols = w.shape
    m_new, u = momentum_step(m, g, hp)
    x = frobenius_normalise(u, hp.ns_eps)
    o = newton_schulz(x, hp.ns_steps, hp.ns_a, hp.ns_b, hp.ns_c)
    w_new = apply_update(w, o, rows, cols, hp)
    return w_new, m_new, o


# ---------------------------------------------------------------------------
# AdamW for the non-matrix tail (Abstract: tensors that are not matrices
# are grouped onto tail owners and optimised with AdamW there)
# ---------------------------------------------------------------------------

def adamw_step(w, g, m1, m2, t: int, hp: Hparams):
    """One AdamW step (bias-corrected moments, decoupled weight decay).

    t is the 1-based step count.  Returns (w_new, m1_new, m2_new), fp64.
    """
    if t < 1:
        raise ValueError("AdamW step count is 1-based")
    w = np.asarray(w, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    m1 = np.asarray(m1, dtype=np.float64)
    m2 = np.asarray(m2, dtype=np.float64)
    b1, b2 = hp.adam_beta1, hp.adam_beta2
    m1_new = b1 * m1 + (1.0 - b1) * g
    m2_new = b2 * m2 + (1.0 - b2) * g * g
    m_hat = m1_new / (1.0 - b1 ** t)
    v_hat = m2_new / (1.0 - b2 ** t)
    w_new = (w * (1.0 - hp.adam_lr * hp.adam_weight_decay)
             - hp.adam_lr * m_hat / (np.sqrt(v_hat) + hp.adam_eps))
    return w_new, m1_new, m2_new


def is_muon_shape(rows: int, cols: int) -> bool:
    """Routing: a tensor with two non-trivial dimensions is a Muon matrix;
    everything else (vectors, scalars) is tail and goes to AdamW."""
    return rows > 1 and cols > 1


# ---------------------------------------------------------------------------
# Storage rounding (every stored tensor is rounded once, to nearest-even)
# ---------------------------------------------------------------------------

def round_to_f32(x) -> np.ndarray:
    """fp64 -> float32 with round-to-nearest-even, returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_bf16(x) -> np.ndarray:
    """fp64 -> bfloat16 with round-to-nearest-even, returned as fp64.

    bfloat16 keeps the float32 exponent and the top 7 fraction bits.  The
    two bfloat16 neighbours of x are found by truncating x's float32 bit
    pattern; the nearer one wins and an exact tie goes to the one with an
    even last bit.  Distances are measured in fp64, so there is no double
    rounding through float32.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    finite = np.isfinite(flat_x)
    flat_o[~finite] = flat_x[~finite]
    xf = flat_x[finite]
    # float32 truncation toward zero keeps the bfloat16 candidate whose
    # magnitude does not exceed |x| (after one float32 rounding step that
    # may move x; handled by checking both neighbours of the truncation).
    bits = xf.astype(np.float32).view(np.uint32)
    base = bits & np.uint32(0xFFFF0000)
    cand = [base.astype(np.int64) + d * 0x10000 for d in (-1, 0, 1)]
    best = None
    best_err = None
    best_even = None
    for cb in cand:
        cb = np.clip(cb, 0, 0xFFFFFFFF).astype(np.uint32)
        val = cb.view(np.float32).astype(np.float64)
        err = np.abs(val - xf)
        even = ((cb >> np.uint32(16)) & np.uint32(1)) == 0
        if best is None:
            best, best_err, best_even = val, err, even
            continue
        better = (err < best_err) | ((err == best_err) & even & ~best_even)
        best = np.where(better, val, best)
        best_err = np.where(better, err, best_err)
        best_even = np.where(better, even, best_even)
    flat_o[finite] = best
    return out


def round_to_dtype(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return round_to_f32(x)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown storage dtype {dtype}")


# ---------------------------------------------------------------------------
# Owner step over a table of whole tensors
# ---------------------------------------------------------------------------

@dataclass
class TensorState:
    """One table entry as plain fp64 arrays, in the entry's own shape.

    For a Muon entry ``state`` is (momentum,); for an AdamW entry it is
    (m1, m2).
    """

    rows: int
    cols: int
    dtype: str
    param: np.ndarray
    grad: np.ndarray
    state: tuple


def owner_step(entries, step: int, hp: Hparams, role_override=None):
    """Run one owner step over every entry, in table order.

    ``entries`` is a list of TensorState.  ``role_override`` may map an
    entry index to "muon" or "adamw"; otherwise the shape decides.  Empty
    entries (rows*cols == 0) are skipped.  Returns a list of dicts with the
    unrounded fp64 results and the storage-rounded ones:
    {"role", "param", "param_stored", "state", "state_stored", "o"}.
    """
    out = []
    for idx, e in enumerate(entries):
        if e.rows * e.cols == 0:
            out.append({"role": "empty"})
            continue
        role = None if role_override is None else role_override.get(idx)
        if role is None:
            role = "muon" if is_muon_shape(e.rows, e.cols) else "adamw"
        if role == "muon":
            w, m, o = muon_matrix_step(e.param, e.grad, e.state[0], hp)
            out.append({
                "role": "muon",
                "param": w,
                "param_stored": round_to_dtype(w, e.dtype),
                "state": (m,),
                "state_stored": (round_to_f32(m),),
                "o": o,
            })
        else:
            w, m1, m2 = adamw_step(e.param, e.grad, e.state[0], e.state[1], step, hp)
            out.append({
                "role": "adamw",
                "param": w,
                "param_stored": round_to_dtype(w, e.dtype),
                "state": (m1, m2),
                "state_stored": (round_to_f32(m1), round_to_f32(m2)),
                "o": None,
            })
    return out
