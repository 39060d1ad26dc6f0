"""Pins of the float64 gate functions (oracle/gates.py) on the CPU.

What pins them, besides the functions themselves:
* hand-derived values (tests/golden/gates_hand.json);
* closed forms: softplus(x) - softplus(-x) = x, softplus(0) = log 2, its
  limits; e^g = (1 + e^(a + bias))^(-e^A) evaluated as a power; silu's
  limits; a one-hot row's norm sqrt(d_v);
* invariants: g <= 0; the per-head parameters follow the head axis; a row's
  norm ignores the other rows and is unchanged by scaling the row (eps = 0);
  the output is odd in o;
* the short convolution: numpy's own convolution of each channel's history
  and rows; one-hot taps (the current row, a shift by W - 1 rows into the
  history); a constant input's partial tap sums; a sequence run in two
  calls, the state carried, equal to one call; packed sequences that do not
  see each other.
Each planted mutation of oracle/gates.py (a dropped factor, a wrong sign, a
swapped axis, an activation exchanged, taps reversed, history lost or taken
from the previous sequence) breaks at least one pin.
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
    for c in GOLDEN["short_conv"]:
        st = None if c["state"] is None else np.asarray(c["state"])
        y, fin = m.short_conv(np.asarray(c["x"]), np.asarray(c["w"]), c["lengths"], st)
        assert np.abs(y - np.asarray(c["y"])).max() <= tol, c["derivation"]
        assert np.abs(fin - np.asarray(c["final"])).max() <= tol, c["derivation"]


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


def _conv_case(rng, lengths, D, W, with_state=True):
    x = rng.normal(0, 1, (sum(lengths), D))
    w = rng.normal(0, 1, (D, W))
    st = rng.normal(0, 1, (len(lengths), W - 1, D)) if with_state else None
    return x, w, st


def pin_conv_numpy(m):
    """Each channel against numpy's convolution of its history and rows
    (np.convolve flips its second argument, so the taps go in reversed)."""
    rng = np.random.default_rng(7)
    for W in (1, 2, 3, 4):
        lengths = [5, 0, 1, 2, 9, 3]
        for with_state in (True, False):
            x, w, st = _conv_case(rng, lengths, 3, W, with_state)
            y, fin = m.short_conv(x, w, lengths, st)
            assert y.shape == x.shape and fin.shape == (len(lengths), W - 1, 3)
            b = 0
            for n, L in enumerate(lengths):
                hist = st[n] if with_state else np.zeros((W - 1, 3))
                e = np.concatenate([hist, x[b:b + L]], axis=0)
                for c in range(3 if L > 0 else 0):  # (np.convolve takes no empty input)
                    want = np.convolve(e[:, c], w[c, ::-1], mode="valid")
                    assert np.allclose(y[b:b + L, c], want, rtol=1e-13, atol=1e-13)
                if W > 1:
                    assert np.array_equal(fin[n], e[len(e) - (W - 1):])
                b += L


def pin_conv_taps(m):
    """One-hot taps: the last tap passes the current row, the first one the
    row W - 1 back (the history for the first W - 1 rows)."""
    rng = np.random.default_rng(8)
    lengths = [6, 2]
    x, _, st = _conv_case(rng, lengths, 4, 4)
    last = np.zeros((4, 4))
    last[:, 3] = 1.0
    y, _ = m.short_conv(x, last, lengths, st)
    assert np.array_equal(y, x)
    first = np.zeros((4, 4))
    first[:, 0] = 1.0
    y, fin = m.short_conv(x, first, lengths, st)
    assert np.array_equal(y[3:6], x[0:3]) and np.array_equal(y[0:3], st[0])
    assert np.array_equal(y[6:8], st[1][0:2])
    assert np.array_equal(fin[0], x[3:6]) and np.array_equal(fin[1], np.concatenate([st[1][2:], x[6:8]]))
    # per-channel taps: channel c keeps only its own weights
    mixed = np.zeros((4, 4))
    for c in range(4):
        mixed[c, c] = 1.0
    y, _ = m.short_conv(x, mixed, [6], None)
    for c in range(4):
        shift = 3 - c
        assert np.array_equal(y[shift:6, c], x[0:6 - shift, c])
        assert np.all(y[:shift, c] == 0.0)


def pin_conv_constant(m):
    """A constant row after zero history: y[t] = sum_{j >= W-1-t} w[:, j]."""
    w = np.array([[0.25, -2.0, 3.0, 0.5], [1.0, 2.0, 4.0, 8.0]])
    y, _ = m.short_conv(np.ones((7, 2)), w, [7], None)
    for t in range(7):
        want = w[:, max(0, 3 - t):].sum(axis=1)
        assert np.allclose(y[t], want, rtol=0, atol=1e-15)


def pin_conv_split_and_packing(m):
    """A sequence in two calls (the first call's final state carried) equals
    one call; packed sequences do not see each other."""
    rng = np.random.default_rng(9)
    x, w, st = _conv_case(rng, [11], 5, 4)
    y, fin = m.short_conv(x, w, [11], st)
    for cut in (0, 1, 2, 3, 7, 11):
        y1, f1 = m.short_conv(x[:cut], w, [cut], st)
        y2, f2 = m.short_conv(x[cut:], w, [11 - cut], f1)
        assert np.allclose(np.concatenate([y1, y2]), y, rtol=0, atol=1e-13)
        assert np.array_equal(f2, fin)
    lengths = [4, 6, 3]
    x, w, st = _conv_case(rng, lengths, 2, 3)
    y, fin = m.short_conv(x, w, lengths, st)
    x2 = x.copy()
    x2[:4] = rng.normal(0, 1, (4, 2))  # sequence 0 changed
    y2, fin2 = m.short_conv(x2, w, lengths, st)
    assert np.array_equal(y2[4:], y[4:]) and np.array_equal(fin2[1:], fin[1:])
    assert not np.allclose(y2[:4], y[:4])


PINS = [pin_golden, pin_softplus, pin_decay, pin_silu, pin_output_gate, pin_conv_numpy,
        pin_conv_taps, pin_conv_constant, pin_conv_split_and_packing]


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
    "conv_taps_reversed": ("y[b + t] += w[:, j] * e[t + j]", "y[b + t] += w[:, W - 1 - j] * e[t + j]"),
    "conv_one_channel_weights": ("y[b + t] += w[:, j] * e[t + j]", "y[b + t] += w[0, j] * e[t + j]"),
    "conv_current_row_dropped": ("for j in range(W):", "for j in range(W - 1):"),
    "conv_history_ignored": ("hist = np.zeros((W - 1, D)) if state is None else _f64(state[n])",
                             "hist = np.zeros((W - 1, D))"),
    "conv_history_from_previous_sequence": (
        "e = np.concatenate([hist, x[b:b + L]], axis=0)",
        "e = np.concatenate([x[b - (W - 1):b] if b >= W - 1 else hist, x[b:b + L]], axis=0)"),
    "conv_final_one_row_early": ("final[n] = e[L:L + W - 1]", "final[n] = e[max(L - 1, 0):max(L - 1, 0) + W - 1]"),
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
        except Exception:  # a failed check, or a mutant that no longer runs
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
