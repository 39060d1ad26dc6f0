"""Pins of the float64 gate functions (oracle/gates.py) on the CPU.

What pins them, besides the functions themselves:
* hand-derived values (tests/golden/gates_hand.json);
* closed forms: softplus(x) - softplus(-x) = x, softplus(0) = log 2, its
  limits; e^g = (1 + e^(a + bias))^(-e^A) evaluated as a power; silu's
  limits; a one-hot row's norm sqrt(d_v);
* invariants: g <= 0; the per-head parameters follow the head axis; a row's
  norm ignores the other rows and is unchanged by scaling the row (eps = 0);
  the output is odd in o.
Each planted mutation of oracle/gates.py (a dropped factor, a wrong sign, a
swapped axis, an activation exchanged) breaks at least one pin.
"""
import json
import math
import os
import types

import numpy as np
import pytest

from oracle import gates

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "gates_hand.json")))
SRC = os.path.join(os.path.dirname(gates.__file__), "gates.py")


def pin_golden(m):
    tol = GOLDEN["tolerance_abs"]
    for c in GOLDEN["decay"]:
        g = m.decay_from_projection(c["a"], c["A"], c["bias"])
        assert abs(float(g) - c["g"]) <= tol, c["derivation"]
    for c in GOLDEN["output_gate"]:
        y = m.output_gate(c["o"], c["z"], c["w"], c["eps"])
        assert np.abs(y - np.asarray(c["y"])).max() <= tol, c["derivation"]


def pin_softplus(m):
    x = np.linspace(-30, 30, 121)
    assert np.allclose(m.softplus(x) - m.softplus(-x), x, rtol=0, atol=1e-12)
    assert abs(m.softplus(0.0) - math.log(2.0)) < 1e-15
    assert abs(m.softplus(40.0) - 40.0) < 1e-12
    assert abs(m.softplus(-40.0) / math.exp(-40.0) - 1.0) < 1e-12
    assert np.all(np.diff(m.softplus(x)) > 0)


def pin_decay(m):
    rng = np.random.default_rng(5)
    T, H = 50, 6
    a = rng.normal(0, 3, (T, H))
    A = rng.normal(0, 1, H)
    b = rng.normal(0, 2, H)
    g = m.decay_from_projection(a, A, b)
    assert g.shape == (T, H) and np.all(g <= 0)
    # alpha = e^g = (1 + e^(a + bias))^(-e^A), evaluated as a power
    alpha = np.power(1.0 + np.exp(a + b), -np.exp(A))
    assert np.allclose(np.exp(g), alpha, rtol=1e-12, atol=0)
    # the per-head parameters follow the head axis
    for h in range(H):
        gh = m.decay_from_projection(a[:, h], A[h], b[h])
        assert np.array_equal(gh, g[:, h])
    # decreasing in the projection
    assert np.all(np.diff(m.decay_from_projection(np.linspace(-5, 5, 11), 0.3, 0.1)) < 0)


def pin_silu(m):
    assert m.silu(0.0) == 0.0
    assert abs(m.silu(40.0) - 40.0) < 1e-12
    assert abs(m.silu(-40.0) / (-40.0 * math.exp(-40.0)) - 1.0) < 1e-12
    assert abs(m.silu(math.log(3.0)) - 0.75 * math.log(3.0)) < 1e-15


def pin_output_gate(m):
    rng = np.random.default_rng(6)
    R, d = 7, 16
    o = rng.normal(0, 1, (R, d))
    z = rng.normal(0, 2, (R, d))
    w = rng.normal(1, 0.3, d)
    y = m.output_gate(o, z, w, 0.0)
    assert y.shape == (R, d)
    # each row's norm is its own
    o2 = o.copy()
    o2[3] *= 10.0
    o2[5] = rng.normal(0, 1, d)
    y2 = m.output_gate(o2, z, w, 0.0)
    keep = [r for r in range(R) if r != 5]
    assert np.allclose(y2[keep], y[keep], rtol=1e-12, atol=1e-15)
    # odd in o
    assert np.allclose(m.output_gate(-o, z, w, 1e-3), -m.output_gate(o, z, w, 1e-3), rtol=0, atol=1e-15)
    # a one-hot row: o / rms = sqrt(d) e_j; with z = 40, silu(z) ~ 40
    for j in (0, 5, d - 1):
        e = np.zeros((1, d))
        e[0, j] = 2.5
        yj = m.output_gate(e, np.full((1, d), 40.0), w, 0.0)
        want = np.zeros((1, d))
        want[0, j] = math.sqrt(d) * w[j] * 40.0
        assert np.allclose(yj, want, rtol=1e-12, atol=1e-12)
    # eps: a row of ones with eps = d_v - 1 ... sqrt(1 + eps)
    ones = np.ones((1, d))
    yo = m.output_gate(ones, np.full((1, d), 40.0), np.ones(d), 3.0)
    assert np.allclose(yo, 0.5 * 40.0, rtol=1e-12)


PINS = [pin_golden, pin_softplus, pin_decay, pin_silu, pin_output_gate]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_gates_pins(pin):
    pin(gates)


MUTATIONS = {
    "softplus_is_exp": ("return np.logaddexp(0.0, _f64(x))", "return np.exp(_f64(x))"),
    "softplus_is_relu": ("return np.logaddexp(0.0, _f64(x))", "return np.maximum(0.0, _f64(x))"),
    "decay_sign": ("return -np.exp(A) * softplus(a + b)", "return np.exp(A) * softplus(a + b)"),
    "rate_not_exponentiated": ("return -np.exp(A) * softplus(a + b)", "return -A * softplus(a + b)"),
    "bias_after_softplus": ("return -np.exp(A) * softplus(a + b)", "return -np.exp(A) * (softplus(a) + b)"),
    "bias_dropped": ("return -np.exp(A) * softplus(a + b)", "return -np.exp(A) * softplus(a)"),
    "silu_is_sigmoid": ("return z * sigmoid(z)", "return sigmoid(z)"),
    "silu_sign": ("return 1.0 / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(z))"),
    "sum_not_mean": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                     "ms = np.sum(o * o, axis=-1, keepdims=True)"),
    "norm_over_rows": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                       "ms = np.mean(o * o, axis=0, keepdims=True)"),
    "eps_outside_root": ("return o / np.sqrt(ms + eps) * w * silu(z)",
                         "return o / (np.sqrt(ms) + eps) * w * silu(z)"),
    "weight_dropped": ("return o / np.sqrt(ms + eps) * w * silu(z)",
                       "return o / np.sqrt(ms + eps) * silu(z)"),
    "gate_dropped": ("return o / np.sqrt(ms + eps) * w * silu(z)",
                     "return o / np.sqrt(ms + eps) * w"),
    "gate_on_output": ("return o / np.sqrt(ms + eps) * w * silu(z)",
                       "return o / np.sqrt(ms + eps) * w * silu(o)"),
    "rms_of_absolute": ("ms = np.mean(o * o, axis=-1, keepdims=True)",
                        "ms = np.mean(np.abs(o), axis=-1, keepdims=True) ** 2"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_gate_mutation_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = types.ModuleType(f"gates_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
