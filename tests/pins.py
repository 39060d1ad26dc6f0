"""Pins of the float64 oracle: facts fixed by the mathematics of the gated
delta rule, each computed WITHOUT calling the oracle's own token loop, so
that a wrong term, sign, index or operand in the oracle fails at least one.

The recurrence (the gated delta rule of the chunked Gated DeltaNet prefill
that "Open-Jev-27B-v1.1 native text worker", section "Validation and
optimization scope", tests against float64 references; the pages print no
formula, so this is the definition the library takes, with the state
written as d_k x d_v):
    H_t = alpha_t (I - b_t k^_t k^_t^T) H_{t-1} + b_t k^_t v_t^T,
    o_t = scale * H_t^T q^_t,   x^ = x / sqrt(|x|^2 + eps),  alpha = exp(g).

Each ``pin_*`` takes the loaded oracle library and returns the largest
violation (a float); ``PIN_TOL`` gives the bound each must stay under.
``tests/test_oracle_pins.py`` asserts them for the real oracle and
``tests/test_oracle_mutations.py`` checks that planted mistakes break one.
"""
from __future__ import annotations

import json
import os

import numpy as np

from oracle import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _norm_rows(x, eps):
    return x / np.sqrt(np.sum(x.astype(np.float64) ** 2, -1, keepdims=True) + eps)


def _f32(x):
    return np.asarray(x, np.float32)


def _run(lib, q, k, v, g, b, lengths, init=None, scale=1.0, eps=1e-6):
    return oracle.reference(_f32(q), _f32(k), _f32(v), _f32(g), _f32(b),
                            lengths, None if init is None else _f32(init),
                            scale=scale, eps=eps, lib=lib, threads=2)


def _rand_case(seed, T, hk, hv, d, g_low=-1.0, init=True, lengths=None,
               dv=None):
    r = _rng(seed)
    dv = d if dv is None else dv
    q = r.standard_normal((T, hk, d)).astype(np.float32)
    k = r.standard_normal((T, hk, d)).astype(np.float32)
    v = r.standard_normal((T, hv, dv)).astype(np.float32)
    g = r.uniform(g_low, 0.0, (T, hv)).astype(np.float32)
    b = r.uniform(0.0, 1.0, (T, hv)).astype(np.float32)
    lengths = lengths or [T]
    H0 = (r.standard_normal((len(lengths), hv, d, dv)).astype(np.float32)
          if init else None)
    return q, k, v, g, b, lengths, H0


def _seq_starts(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(int)


# ---------------------------------------------------------------- closed forms

def pin_decay_beta0(lib):
    """b = 0 removes every write: H_t = e^{g_1+..+g_t} H_0 and
    o_t = scale e^{gamma_t} H_0^T q^_t (per sequence, per value head, with
    value head h reading key head h // (Hv/Hk))."""
    d, hk, hv, lens = 6, 2, 4, [5, 7]
    q, k, v, g, b, lengths, H0 = _rand_case(11, sum(lens), hk, hv, d,
                                            g_low=-0.7, lengths=lens)
    b[:] = 0.0
    scale, eps = 0.75, 1e-6
    out, fin = _run(lib, q, k, v, g, b, lengths, H0, scale=scale, eps=eps)
    qn = _norm_rows(q.astype(np.float64), eps)
    err = 0.0
    st = _seq_starts(lengths)
    for i in range(len(lengths)):
        for h in range(hv):
            kh = h // (hv // hk)
            gam = np.cumsum(g[st[i]:st[i + 1], h].astype(np.float64))
            for j, t in enumerate(range(st[i], st[i + 1])):
                exp_o = scale * np.exp(gam[j]) * (H0[i, h].T.astype(np.float64) @ qn[t, kh])
                err = max(err, np.abs(out[t, h] - exp_o).max())
            err = max(err, np.abs(fin[i, h] - np.exp(gam[-1]) * H0[i, h]).max())
    return err


def pin_identity_alpha1_beta0(lib):
    """alpha = 1 and b = 0 (the literal reading of 'alpha=1 with beta=0'):
    the state never changes, o_t = H_0^T q^_t and the final state is H_0."""
    d, T = 5, 6
    q, k, v, g, b, lengths, H0 = _rand_case(12, T, 1, 1, d)
    g[:] = 0.0
    b[:] = 0.0
    out, fin = _run(lib, q, k, v, g, b, lengths, H0, eps=0.0)
    qn = _norm_rows(q.astype(np.float64), 0.0)
    exp_o = np.einsum("ij,ti->tj", H0[0, 0].astype(np.float64), qn[:, 0])
    return max(np.abs(out[:, 0] - exp_o).max(), np.abs(fin[0, 0] - H0[0, 0]).max())


def pin_orthonormal_keys(lib):
    """Mutually orthogonal keys make every (I - b k^k^T) act on its own key
    only, so from H_0 = 0 the rule is gated linear attention exactly:
    o_t = scale sum_{s<=t} b_s e^{gamma_t - gamma_s} (q^_t . k^_s) v_s and
    H_T = sum_s b_s e^{gamma_T - gamma_s} k^_s v_s^T."""
    d, T = 8, 8
    r = _rng(13)
    # Sylvester-Hadamard rows: +-1 entries, exactly orthogonal in floating
    # point; power-of-two row scales keep them exact in float32.
    Hd = np.array([[1.0]])
    while Hd.shape[0] < d:
        Hd = np.block([[Hd, Hd], [Hd, -Hd]])
    scales = 2.0 ** r.integers(-2, 3, (T, 1))
    k = (Hd[r.permutation(d)[:T]] * scales)[:, None, :].astype(np.float32)
    q = r.standard_normal((T, 1, d)).astype(np.float32)
    v = r.standard_normal((T, 1, d)).astype(np.float32)
    g = r.uniform(-1.0, 0.0, (T, 1)).astype(np.float32)
    b = r.uniform(0.0, 1.0, (T, 1)).astype(np.float32)
    scale = 1.3
    out, fin = _run(lib, q, k, v, g, b, [T], None, scale=scale, eps=0.0)
    qn = _norm_rows(q[:, 0].astype(np.float64), 0.0)
    kn = _norm_rows(k[:, 0].astype(np.float64), 0.0)
    gam = np.cumsum(g[:, 0].astype(np.float64))
    err = 0.0
    for t in range(T):
        acc = np.zeros(d)
        for s in range(t + 1):
            acc += b[s, 0] * np.exp(gam[t] - gam[s]) * (qn[t] @ kn[s]) * v[s, 0]
        err = max(err, np.abs(out[t, 0] - scale * acc).max())
    HT = sum(b[s, 0] * np.exp(gam[-1] - gam[s]) * np.outer(kn[s], v[s, 0])
             for s in range(T))
    return max(err, np.abs(fin[0, 0] - HT).max())


def pin_linear_attention_first_order(lib):
    """alpha = 1, b = beps small, H_0 = 0: o_t / beps approaches cumulative
    linear attention sum_{s<=t} (q^_t . k^_s) v_s with error O(beps t).
    Returned value: the relative deviation divided by beps * T (order 1 for
    a correct recurrence, order 1/beps for a wrong one)."""
    d, T, beps = 6, 9, 1e-6
    q, k, v, g, b, lengths, _ = _rand_case(14, T, 1, 1, d, init=False)
    g[:] = 0.0
    b[:] = beps
    out, _ = _run(lib, q, k, v, g, b, lengths, None, eps=0.0)
    qn = _norm_rows(q[:, 0].astype(np.float64), 0.0)
    kn = _norm_rows(k[:, 0].astype(np.float64), 0.0)
    b32 = float(np.float32(beps))
    worst = 0.0
    for t in range(T):
        la = sum((qn[t] @ kn[s]) * v[s, 0].astype(np.float64) for s in range(t + 1))
        rel = np.abs(out[t, 0] / b32 - la).max() / max(np.abs(la).max(), 1e-12)
        worst = max(worst, rel / (b32 * T))
    return worst


def pin_beta1_overwrite(lib):
    """b = 1 writes v_t exactly along k^_t: k^_t^T H_t = v_t^T for any alpha
    and H_{t-1}; with q = k the output is o_t = v_t (scale 1, eps 0)."""
    d, hk, hv, lens = 7, 1, 3, [4, 6]
    q, k, v, g, b, lengths, H0 = _rand_case(15, sum(lens), hk, hv, d, lengths=lens)
    b[:] = 1.0
    out, _ = _run(lib, k, k, v, g, b, lengths, H0, eps=0.0)
    return np.abs(out - v.astype(np.float64)).max()


def pin_small_norm_rows(lib):
    """The L2 normalisation is x / sqrt(|x|^2 + eps): one token, H_0 = 0,
    q = k = c e_1 gives o = b (q^ . k^) v = b c^2 / (c^2 + eps) v."""
    d, eps, c = 4, 1e-4, 1e-2
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = c
    v = np.array([[[1.0, -2.0, 3.0, 0.5]]], np.float32)
    g = np.array([[-0.3]], np.float32)
    b = np.array([[0.6]], np.float32)
    out, fin = _run(lib, q, q, v, g, b, [1], None, eps=eps)
    c32, b32 = float(np.float32(c)), float(np.float32(b[0, 0]))
    v64 = v[0, 0].astype(np.float64)
    ratio = c32 * c32 / (c32 * c32 + eps)
    e1 = np.abs(out[0, 0] - b32 * ratio * v64).max()
    kh = c32 / np.sqrt(c32 * c32 + eps)
    e2 = np.abs(fin[0, 0, 0] - b32 * kh * v64).max()
    return max(e1, e2)


def pin_golden_two_token(lib):
    """The hand-derived example in tests/golden/two_token_d2.json."""
    with open(os.path.join(GOLDEN, "two_token_d2.json")) as f:
        gold = json.load(f)
    x = gold["inputs"]
    out, fin = _run(lib, x["q"], x["k"], x["v"], x["g"], x["beta"],
                    x["lengths"], None, scale=x["scale"], eps=x["eps"])
    e = gold["expected"]
    return max(np.abs(out - np.array(e["out"])).max(),
               np.abs(fin - np.array(e["final_state"])).max())


# ------------------------------------------------------- brute-force matrix form

def brute_force(q, k, v, g, b, lengths, H0, scale, eps):
    """Unrolled matrix form with explicit d_k x d_k transitions
    A_t = alpha_t (I - b_t k^_t k^_t^T):
        H_t = (A_t ... A_1) H_0 + sum_{s<=t} (A_t ... A_{s+1}) b_s k^_s v_s^T.
    Quadratic in T; for T <= 8."""
    T, hk, d = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hk
    out = np.zeros((T, hv, dv))
    fin = np.zeros((len(lengths), hv, d, dv))
    st = _seq_starts(lengths)
    for i in range(len(lengths)):
        for h in range(hv):
            kh = h // grp
            rows = range(st[i], st[i + 1])
            kn = {t: k[t, kh].astype(np.float64) / np.sqrt(np.sum(k[t, kh].astype(np.float64) ** 2) + eps) for t in rows}
            qn = {t: q[t, kh].astype(np.float64) / np.sqrt(np.sum(q[t, kh].astype(np.float64) ** 2) + eps) for t in rows}
            A = {t: np.exp(np.float64(g[t, h])) * (np.eye(d) - np.float64(b[t, h]) * np.outer(kn[t], kn[t])) for t in rows}

            def prod(a, z):  # A_z ... A_a  (identity when a > z)
                M = np.eye(d)
                for t in range(a, z + 1):
                    M = A[t] @ M
                return M
            base = np.zeros((d, dv)) if H0 is None else H0[i, h].astype(np.float64)
            Ht = base
            for t in rows:
                Ht = prod(st[i], t) @ base
                for s in range(st[i], t + 1):
                    Ht = Ht + prod(s + 1, t) @ (np.float64(b[s, h]) * np.outer(kn[s], v[s, h].astype(np.float64)))
                out[t, h] = scale * Ht.T @ qn[t]
            fin[i, h] = Ht
    return out, fin


def pin_brute_force(lib):
    """Token loop == unrolled product form on short packed sequences with
    grouped heads (Hv = 2 Hk), a random initial state and d_k != d_v."""
    d, hk, hv, lens = 5, 2, 4, [3, 8, 1]
    q, k, v, g, b, lengths, H0 = _rand_case(16, sum(lens), hk, hv, d,
                                            lengths=lens, dv=3)
    scale, eps = 0.9, 1e-6
    out, fin = _run(lib, q, k, v, g, b, lengths, H0, scale=scale, eps=eps)
    bo, bfin = brute_force(q, k, v, g, b, lengths, H0, scale, eps)
    return max(np.abs(out - bo).max(), np.abs(fin - bfin).max())


PINS = {
    "decay_beta0": pin_decay_beta0,
    "identity_alpha1_beta0": pin_identity_alpha1_beta0,
    "orthonormal_keys": pin_orthonormal_keys,
    "linear_attention_first_order": pin_linear_attention_first_order,
    "beta1_overwrite": pin_beta1_overwrite,
    "small_norm_rows": pin_small_norm_rows,
    "golden_two_token": pin_golden_two_token,
    "brute_force": pin_brute_force,
}

PIN_TOL = {
    "decay_beta0": 1e-12,
    "identity_alpha1_beta0": 1e-12,
    "orthonormal_keys": 1e-12,
    "linear_attention_first_order": 10.0,
    "beta1_overwrite": 1e-12,
    "small_norm_rows": 1e-12,
    "golden_two_token": 1e-6,
    "brute_force": 1e-12,
}
