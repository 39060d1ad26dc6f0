"""Float64 gates on either side of the prefill -- TEST INFRASTRUCTURE.

Only ``tests/`` (and the package smoke check) may import this module.  It
shares nothing with the HIP package.

The serving pages run "fused norm, activation" operations around the chunked
Gated DeltaNet and keep the bf16 rounding points of the unfused sequence when
they fuse a gate into an epilogue ("Open-Jev-27B-v1.1 native text worker",
section "Validation and optimization scope").  They print no formula for
either side, so the two functions below are this library's reading, the
plainest one the rest supports:

* The decay gate from a raw projection a (one value per token and value
  head).  The recurrence needs g <= 0 (alpha = e^g in (0, 1]); a positive
  per-head rate e^A times a softplus of the shifted projection gives that
  for every a:

      g[t, h] = -exp(A[h]) * softplus(a[t, h] + bias[h]),
      softplus(x) = log(1 + e^x).

  (A = 0, bias = 0 and a -> -a give g = log(sigmoid(a)), the gate with no
  per-head parameters.)

* The gated output norm after the prefill.  For each (token, value head)
  row o of d_v outputs, its gate projection row z and a per-channel weight
  w[d_v]:

      y = o / sqrt(mean(o^2) + eps) * w * silu(z),   silu(z) = z / (1 + e^-z)

  The library applies it to the outputs as the prefill stores them (rounded
  to the output type) and rounds y once.

* The short convolution before the activation (the pages name none; this
  is the one a Gated DeltaNet layer runs on its q, k, v projections before
  the SiLU, taken as this library's reading).  Each channel of q, k and v
  (one column of the [T, H * d] token rows) passes through a causal
  depthwise convolution of width W along the tokens of its own sequence:

      y[t, c] = sum_{j=0}^{W-1} w[c, j] * e[t + j, c],

  where e is the sequence's W - 1 history rows (the raw rows before its
  first token; zeros for a fresh sequence) followed by its own rows, so the
  last tap w[c, W-1] multiplies the current token.  The state a later call
  continues from is the last W - 1 rows of e (raw values, not convolved).

Pins: ``tests/test_oracle_gates.py`` (closed forms, hand-derived values in
``tests/golden/gates_hand.json``, invariants, numpy's convolution for the
short convolution) and planted mutations of this file that each break at
least one of them.
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def softplus(x):
    """log(1 + e^x), as log(e^0 + e^x) (numpy's logaddexp, no overflow)."""
    return np.logaddexp(0.0, _f64(x))


def decay_from_projection(a, a_log, bias):
    """g = -exp(A) * softplus(a + bias); a [..., Hv], A and bias [Hv]."""
    a = _f64(a)
    A = _f64(a_log)
    b = _f64(bias)
    return -np.exp(A) * softplus(a + b)


def sigmoid(z):
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    z = _f64(z)
    return z * sigmoid(z)


def output_gate(o, z, w, eps):
    """y = o / sqrt(mean(o^2) + eps) * w * silu(z) over the last axis."""
    o = _f64(o)
    z = _f64(z)
    w = _f64(w)
    ms = np.mean(o * o, axis=-1, keepdims=True)
    return o / np.sqrt(ms + eps) * w * silu(z)


def short_conv(x, w, lengths, state=None):
    """Causal depthwise convolution along the tokens of each sequence.

    x [T, D]: the rows of the sequences back to back, lengths[n] rows each;
    w [D, W]; state [N, W - 1, D]: the raw rows before each sequence (None:
    zeros).  Returns (y [T, D], final [N, W - 1, D]).
    """
    x = _f64(x)
    w = _f64(w)
    D, W = w.shape
    y = np.zeros(x.shape)
    final = np.zeros((len(lengths), W - 1, D))
    b = 0
    for n, L in enumerate(lengths):
        hist = np.zeros((W - 1, D)) if state is None else _f64(state[n])
        e = np.concatenate([hist, x[b:b + L]], axis=0)
        for t in range(L):
            for j in range(W):
                y[b + t] += w[:, j] * e[t + j]
        final[n] = e[L:L + W - 1]
        b += L
    return y, final
