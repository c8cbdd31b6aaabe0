"""Pins for the fp64 oracle: each test ties the oracle to something other
than itself (a closed form, an invariant, an exact special case, a brute
force), so that a plausible slip in the oracle (a dropped term, a wrong sign,
a transposed operand, a missing normalisation) fails at least one of them.
No GPU is needed.
"""

import math

import numpy as np
import pytest

from oracle import muon_oracle as orc

HP = orc.Hparams()
A, B, C = HP.ns_a, HP.ns_b, HP.ns_c


def p5(sigma, steps=5):
    """Scalar recursion of the quintic: the closed form of Newton-Schulz on
    one singular value."""
    s = np.asarray(sigma, dtype=np.float64)
    for _ in range(steps):
        s = A * s + B * s ** 3 + C * s ** 5
    return s


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --- Newton-Schulz against the SVD closed form -----------------------------

@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (8, 8), (1, 7), (16, 32), (32, 16), (64, 128), (37, 53)])
@pytest.mark.parametrize("steps", [0, 1, 2, 5])
def test_ns_matches_svd_closed_form(shape, steps):
    """NS acts on singular values alone: X = U S V^T gives U p^k(S) V^T."""
    x = rand(shape, 11 + shape[0])
    x = x / np.linalg.norm(x)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    want = (u * p5(s, steps)) @ vt
    got = orc.newton_schulz(x, steps, A, B, C)
    assert got.shape == x.shape
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel <= 1e-12, rel


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (16, 40), (33, 20)])
@pytest.mark.parametrize("steps", [0, 1, 2, 3])
def test_ns_apply_matches_svd_closed_form(shape, steps):
    """The vector-applied iteration gives U p^k(S) V^T @ V for a block V."""
    x = rand(shape, 3 + shape[1])
    x = x / np.linalg.norm(x)
    v = rand((shape[1], 3), 99)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    want = ((u * p5(s, steps)) @ vt) @ v
    got = orc.newton_schulz_apply(x, v, steps, A, B, C)
    assert np.linalg.norm(got - want) <= 1e-12 * np.linalg.norm(want)


def test_ns_singular_vectors_unchanged():
    x = rand((24, 40), 3)
    x = x / np.linalg.norm(x)
    u, s, vt = np.linalg.svd(x, full_matrices=False)
    o = orc.newton_schulz(x, 5, A, B, C)
    d = u.T @ o @ vt.T
    off = d - np.diag(np.diag(d))
    assert np.linalg.norm(off) <= 1e-12 * np.linalg.norm(d)
    np.testing.assert_allclose(np.diag(d), p5(s), rtol=1e-12, atol=1e-14)


def test_ns_output_band():
    """Singular values in (0, 1] map into (0, 1.20237]; inputs >= 2e-3 land
    in [0.68182, 1.20237] (ends of the quintic's band after 5 steps)."""
    x = rand((48, 96), 5)
    x = x / np.linalg.norm(x)
    s_in = np.linalg.svd(x, compute_uv=False)
    s_out = np.linalg.svd(orc.newton_schulz(x, 5, A, B, C), compute_uv=False)
    np.testing.assert_allclose(np.sort(s_out), np.sort(p5(s_in)), rtol=1e-11, atol=1e-13)
    assert s_out.max() <= 1.20237 + 1e-6
    big = s_in >= 2e-3
    assert big.any()
    assert np.all(p5(s_in[big]) >= 0.68182 - 1e-6)


def test_ns_transpose_symmetry_by_direct_tall_evaluation():
    """For a tall X the oracle transposes.  Evaluate the tall matrix directly
    with the large Gram X^T X acting from the right instead:
    (aI + b XX^T + c(XX^T)^2) X = X (aI + b X^T X + c (X^T X)^2)."""
    x = rand((40, 12), 9)
    x = x / np.linalg.norm(x)
    y = x.copy()
    for _ in range(5):
        g = y.T @ y
        y = A * y + y @ (B * g + C * g @ g)
    got = orc.newton_schulz(x, 5, A, B, C)
    assert np.linalg.norm(got - y) <= 1e-13 * np.linalg.norm(y)
    np.testing.assert_allclose(orc.newton_schulz(x.T, 5, A, B, C), got.T, rtol=0, atol=1e-14)


# --- Exact special cases of the whole Muon step ----------------------------

def _step_one(w, g, m=None, hp=HP):
    m = np.zeros_like(g) if m is None else m
    return orc.muon_matrix_step(w, g, m, hp)


def test_zero_gradient_gives_pure_weight_decay():
    w = rand((16, 24), 1) * 0.02
    w1, m1, o = _step_one(w, np.zeros((16, 24)))
    assert np.all(o == 0.0)
    assert np.all(m1 == 0.0)
    np.testing.assert_array_equal(w1, w * (1.0 - HP.lr * HP.weight_decay))


def test_rank_one_gradient():
    """G = x y^T has one singular value; after normalisation it is
    ||U||/(||U||+eps), and O = p^5(that) * xhat yhat^T."""
    rng = np.random.default_rng(4)
    x, y = rng.standard_normal(10), rng.standard_normal(14)
    g = np.outer(x, y)
    _, _, o = _step_one(np.zeros((10, 14)), g)
    nrm = (1.0 + HP.momentum) * np.linalg.norm(g)
    sigma = nrm / (nrm + HP.ns_eps)
    want = p5(sigma) * np.outer(x / np.linalg.norm(x), y / np.linalg.norm(y))
    np.testing.assert_allclose(o, want, rtol=1e-12, atol=1e-15)
    # with the decimal coefficients the recursion gives p^5(1) = 0.696436409469752;
    # the float32 coefficients the ABI carries move it by ~3e-8
    s = 1.0
    for _ in range(5):
        s = 3.4445 * s - 4.7750 * s ** 3 + 2.0315 * s ** 5
    assert abs(s - 0.696436409469752) < 1e-14
    assert abs(p5(1.0) - s) < 1e-7


@pytest.mark.parametrize("r,cols", [(4, 9), (16, 20), (64, 64), (9, 4)])
def test_identity_block_gradient(r, cols):
    """G = [I_r 0] has r singular values 1, normalised to 1/sqrt(r) (eps
    included), so O = p^5(1/sqrt(r)) [I_r 0] (or its transpose when tall)."""
    rows = r
    if r > cols:  # tall: [I; 0]
        rows, r = r, cols
        g = np.zeros((rows, cols))
        g[:r, :r] = np.eye(r)
    else:
        g = np.zeros((rows, cols))
        g[:r, :r] = np.eye(r)
    _, _, o = _step_one(np.zeros_like(g), g)
    nrm = (1.0 + HP.momentum) * math.sqrt(r)
    sigma = (1.0 + HP.momentum) / (nrm + HP.ns_eps)
    np.testing.assert_allclose(o, p5(sigma) * g, rtol=1e-12, atol=1e-15)


def test_scale_invariance():
    """NS(alpha U) = NS(U) up to eps/||U||."""
    g = rand((20, 30), 8)
    _, _, o1 = _step_one(np.zeros_like(g), g)
    _, _, o2 = _step_one(np.zeros_like(g), 1e-3 * g)
    bound = 10 * HP.ns_eps / np.linalg.norm((1 + HP.momentum) * 1e-3 * g)
    assert np.linalg.norm(o1 - o2) / np.linalg.norm(o1) < bound
    # with eps = 0 the invariance is exact up to rounding
    hp0 = orc.Hparams(ns_eps=0.0)
    _, _, p1 = _step_one(np.zeros_like(g), g, hp=hp0)
    _, _, p2 = _step_one(np.zeros_like(g), 1e-3 * g, hp=hp0)
    assert np.linalg.norm(p1 - p2) / np.linalg.norm(p1) < 1e-13


def test_momentum_closed_forms():
    """From zero momentum: M1 = G1 and U1 = (1+beta) G1, so O1 = NS(G1/||G1||).
    Step 2: M2 = beta G1 + G2, U2 = G2 + beta M2."""
    beta = HP.momentum
    g1, g2 = rand((12, 18), 21), rand((12, 18), 22)
    w = rand((12, 18), 23) * 0.02
    w1, m1, o1 = _step_one(w, g1)
    np.testing.assert_array_equal(m1, g1)
    u1 = (1 + beta) * g1
    x1 = u1 / (np.linalg.norm(u1) + HP.ns_eps)
    u, s, vt = np.linalg.svd(x1, full_matrices=False)
    np.testing.assert_allclose(o1, (u * p5(s)) @ vt, rtol=1e-9, atol=1e-12)
    w2, m2, o2 = orc.muon_matrix_step(w1, g2, m1, HP)
    np.testing.assert_allclose(m2, beta * g1 + g2, rtol=1e-15, atol=0)
    u2 = g2 + beta * (beta * g1 + g2)
    u, s, vt = np.linalg.svd(u2 / (np.linalg.norm(u2) + HP.ns_eps), full_matrices=False)
    np.testing.assert_allclose(o2, (u * p5(s)) @ vt, rtol=1e-9, atol=1e-12)


def test_plain_momentum_without_nesterov():
    hp = orc.Hparams(nesterov=False)
    g1 = rand((8, 8), 2)
    _, m1, _ = orc.muon_matrix_step(np.zeros((8, 8)), g1, np.zeros((8, 8)), hp)
    g2 = rand((8, 8), 3)
    _, _, o2 = orc.muon_matrix_step(np.zeros((8, 8)), g2, m1, hp)
    u = hp.momentum * g1 + g2
    uu, s, vt = np.linalg.svd(u / (np.linalg.norm(u) + hp.ns_eps))
    np.testing.assert_allclose(o2, (uu * p5(s)) @ vt, rtol=1e-9, atol=1e-12)


def test_update_uses_scale_and_decoupled_decay():
    """W1 = W (1 - lr wd) - lr * scale * O with scale from the literal shape."""
    g = rand((30, 10), 5)  # tall: scale sqrt(3)
    w = rand((30, 10), 6) * 0.02
    w1, _, o = _step_one(w, g)
    np.testing.assert_allclose(
        w1, w * (1 - HP.lr * HP.weight_decay) - HP.lr * math.sqrt(3.0) * o, rtol=1e-15, atol=1e-17)
    # tall O has orthonormal-ish columns: O^T O = V p^5(S)^2 V^T
    u = (1 + HP.momentum) * g
    s = np.linalg.svd(u / (np.linalg.norm(u) + HP.ns_eps), compute_uv=False)
    np.testing.assert_allclose(np.sort(np.linalg.svd(o, compute_uv=False)), np.sort(p5(s)), rtol=1e-11)


def test_lr_shape_scale_conventions():
    assert orc.lr_shape_scale(768, 2304, 0) == 1.0
    assert orc.lr_shape_scale(3072, 768, 0) == 2.0
    assert orc.lr_shape_scale(4096, 4096, 0) == 1.0
    assert orc.lr_shape_scale(14336, 4096, 0) == math.sqrt(3.5)
    assert orc.lr_shape_scale(1024, 4096, 1) == pytest.approx(0.2 * 64.0)


def test_ns_zero_steps_is_normalised_input():
    g = rand((5, 7), 2)
    _, _, o = orc.muon_matrix_step(np.zeros((5, 7)), g, np.zeros((5, 7)), orc.Hparams(ns_steps=0))
    u = (1 + HP.momentum) * g
    np.testing.assert_allclose(o, u / (np.linalg.norm(u) + HP.ns_eps), rtol=1e-15)


# --- AdamW -----------------------------------------------------------------

def test_adamw_step_one_closed_form():
    """At t = 1 the bias-corrected moments are g and g^2 exactly, so
    W1 = W0 (1 - lr wd) - lr g / (|g| + eps)."""
    g = rand(1000, 7) * 1e-3
    w = rand(1000, 8)
    w1, m1, m2 = orc.adamw_step(w, g, np.zeros(1000), np.zeros(1000), 1, HP)
    want = w * (1 - HP.adam_lr * HP.adam_weight_decay) - HP.adam_lr * g / (np.abs(g) + HP.adam_eps)
    np.testing.assert_allclose(w1, want, rtol=1e-13, atol=1e-18)
    np.testing.assert_allclose(m1, (1 - HP.adam_beta1) * g, rtol=1e-15)
    np.testing.assert_allclose(m2, (1 - HP.adam_beta2) * g * g, rtol=1e-15)


def test_adamw_constant_gradient_bias_correction_exact():
    """With a constant gradient the bias-corrected moments equal g and g^2 at
    every step, so each step is the step-1 update again."""
    g = rand(64, 9)
    w = rand(64, 10)
    m1 = np.zeros(64)
    m2 = np.zeros(64)
    for t in range(1, 6):
        w_prev = w
        w, m1, m2 = orc.adamw_step(w, g, m1, m2, t, HP)
        want = w_prev * (1 - HP.adam_lr * HP.adam_weight_decay) - HP.adam_lr * g / (np.abs(g) + HP.adam_eps)
        np.testing.assert_allclose(w, want, rtol=1e-12, atol=1e-15)


def test_adamw_rejects_zero_step():
    with pytest.raises(ValueError):
        orc.adamw_step(np.zeros(2), np.zeros(2), np.zeros(2), np.zeros(2), 0, HP)


# --- Storage rounding ------------------------------------------------------

def _all_bf16_values():
    bits = np.arange(0, 1 << 16, dtype=np.uint32) << np.uint32(16)
    vals = bits.view(np.float32).astype(np.float64)
    return vals[np.isfinite(vals)]


def test_bf16_rounding_against_exhaustive_nearest():
    """Brute force: the nearest of all finite bfloat16 values, ties to the
    one whose last kept bit is even."""
    table = np.unique(_all_bf16_values())
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(3000) * 0.02,
        rng.standard_normal(1000) * 1e-30,
        rng.standard_normal(1000) * 1e4,
        # exact midpoints between neighbouring bf16 values, and near-midpoints
        (table[1000:1400] + table[1001:1401]) / 2,
        (table[30000:30200] + table[30001:30201]) / 2 * (1 + 1e-12),
        (table[40000:40200] + table[40001:40201]) / 2 * (1 - 1e-12),
    ])
    got = orc.round_to_bf16(x)
    idx = np.clip(np.searchsorted(table, x), 1, len(table) - 1)
    lo, hi = table[idx - 1], table[idx]
    dlo, dhi = np.abs(x - lo), np.abs(hi - x)
    hi_bits = hi.astype(np.float32).view(np.uint32)
    hi_even = ((hi_bits >> 16) & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(hi_even, hi, lo)))
    # signed zero compares equal; compare values
    np.testing.assert_array_equal(got, want)


def test_f32_rounding_is_float32_cast():
    x = np.array([0.1, 1 / 3, 2.0 ** -140, -7.25])
    np.testing.assert_array_equal(orc.round_to_f32(x), np.array([np.float32(v) for v in x], dtype=np.float64))


# --- Table routing ---------------------------------------------------------

def test_owner_step_routes_and_skips_empty():
    rng = np.random.default_rng(1)
    ents = [
        orc.TensorState(4, 6, "f32", rng.standard_normal((4, 6)), rng.standard_normal((4, 6)), (np.zeros((4, 6)),)),
        orc.TensorState(1, 5, "f32", rng.standard_normal((1, 5)), rng.standard_normal((1, 5)), (np.zeros((1, 5)), np.zeros((1, 5)))),
        orc.TensorState(0, 5, "bf16", np.zeros((0, 5)), np.zeros((0, 5)), ()),
    ]
    res = orc.owner_step(ents, 1, HP)
    assert [r["role"] for r in res] == ["muon", "adamw", "empty"]
    w_want, _, _ = orc.adamw_step(ents[1].param, ents[1].grad, np.zeros((1, 5)), np.zeros((1, 5)), 1, HP)
    np.testing.assert_array_equal(res[1]["param"], w_want)
