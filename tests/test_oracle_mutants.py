"""Sensitivity of the oracle pins: plant a plausible mistake in a copy of
the oracle's source (on the CPU, in memory) and require that at least one
pin in test_oracle_pins fails against the mutant.  The real oracle file is
never modified.
"""

import importlib.util
import inspect
import sys
import types

import pytest

import tests.test_oracle_pins as pins
from oracle import muon_oracle

MUTANTS = {
    "drop_quintic_term": ("poly = b * gram + c * (gram @ gram)", "poly = b * gram"),
    "wrong_sign_b": ("poly = b * gram + c", "poly = -b * gram + c"),
    "gram_transposed": ("gram = xw @ xw.T", "gram = xw.T @ xw"),
    "update_operand_order": ("xw = a * xw + poly @ xw", "xw = a * (xw + poly @ xw)"),
    "no_normalisation": ("return u / (math.sqrt(float(np.sum(u * u))) + eps)", "return u"),
    "eps_inside_sqrt": ("math.sqrt(float(np.sum(u * u))) + eps", "math.sqrt(float(np.sum(u * u)) + eps)"),
    "nesterov_uses_old_momentum": ("u = g + beta * m_new if", "u = g + beta * m if"),
    "apply_drops_cubic": ("return a * z + b * az + c * _gram(k, az)", "return a * z + c * _gram(k, az)"),
    "apply_transpose_side": ("return bwd(k - 1, _poly(k - 1, w))", "return bwd(k - 1, w)"),
    "ema_momentum": ("m_new = beta * m + g", "m_new = beta * m + (1.0 - beta) * g"),
    "decay_not_lr_scaled": ("w * (1.0 - hp.lr * hp.weight_decay)", "w * (1.0 - hp.weight_decay)"),
    "shape_scale_inverted": ("max(1.0, rows / cols)", "max(1.0, cols / rows)"),
    "adam_no_bias_correction": ("m_hat = m1_new / (1.0 - b1 ** t)", "m_hat = m1_new"),
    "adam_eps_inside_sqrt": ("np.sqrt(v_hat) + hp.adam_eps", "np.sqrt(v_hat + hp.adam_eps)"),
    "adam_beta_swapped": ("m2_new = b2 * m2 + (1.0 - b2) * g * g", "m2_new = b1 * m2 + (1.0 - b1) * g * g"),
    "bf16_ties_to_odd": ("& even & ~best_even", "& ~even & best_even"),
    "ns_one_step_short": ("for _ in range(steps):\n        gram", "for _ in range(steps - 1):\n        gram"),
    "routing_vectors_to_muon": ("return rows > 1 and cols > 1", "return rows >= 1 and cols > 1"),
}


def _mutant_module(old: str, new: str) -> types.ModuleType:
    src = inspect.getsource(muon_oracle)
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    mod.__dict__["__name__"] = "oracle_mutant"
    sys.modules["oracle_mutant"] = mod  # dataclasses resolve their module by name
    try:
        exec(compile(src, "<oracle_mutant>", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


def _pin_cases():
    cases = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            cases.append((fn, {}))
            continue
        # expand the cartesian product of parametrize marks (first few values)
        combos = [{}]
        for m in params:
            names = [n.strip() for n in m.args[0].split(",")]
            new = []
            for c in combos:
                for v in m.args[1][:3]:
                    vals = v if len(names) > 1 else (v,)
                    d = dict(c)
                    d.update(zip(names, vals))
                    new.append(d)
            combos = new
        cases.extend((fn, c) for c in combos)
    return cases


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_some_pin_catches_mutant(mutant, monkeypatch):
    old, new = MUTANTS[mutant]
    mod = _mutant_module(old, new)
    monkeypatch.setattr(pins, "orc", mod)
    monkeypatch.setattr(pins, "HP", mod.Hparams())
    caught = []
    for fn, kwargs in _pin_cases():
        try:
            fn(**kwargs)
        except Exception:  # an assertion or a shape error: the pin fired
            caught.append(fn.__name__)
    assert caught, f"no pin detects mutant {mutant}"


def test_unmutated_copy_passes_every_pin(monkeypatch):
    mod = _mutant_module("import math", "import math")
    monkeypatch.setattr(pins, "orc", mod)
    for fn, kwargs in _pin_cases():
        fn(**kwargs)
