"""Float64 chunked evaluator of the Gated DeltaNet prefill -- TEST INFRASTRUCTURE.

Only ``tests/`` (and the package smoke check) may import this module.  It is
a second, independent float64 route to the same result as the token
recurrence in ``gdn_oracle.c``, written in numpy, and it exposes the
per-chunk intermediates that the GPU stages produce so that each stage can be
checked on its own.

The chunk algebra is the WY (compact product) form of the gated delta
rule: the product over a chunk of the per-token maps
H -> alpha_t (I - beta_t k^ k^T) H + beta_t k^ v^T, written with one
triangular inverse per chunk (derived here from the recurrence in
``gdn_oracle.c``; the pages print no chunk algebra).  For one chunk of n
tokens entering with state H (d_k x d_v), with r, s = 0..n-1 and s <= r
meaning "not after":

    gamma_r = g_0 + ... + g_r                       (chunk-local cumulative gate)
    D_rs    = exp(gamma_r - gamma_s) if s <= r else 0
    A_rs    = beta_r D_rs (k^_r . k^_s)  for s < r, else 0
    T       = (I + A)^-1
    W       = T diag(beta e^gamma) K^,   U~ = T diag(beta) V
    U       = U~ - W H
    P_rs    = scale D_rs (q^_r . k^_s)
    O       = scale diag(e^gamma) Q^ H + P U
    H'      = e^{gamma_last} H + K~^T U,   K~_r = e^{gamma_last - gamma_r} k^_r

Two quantities are regrouped from the same terms:
    Q' = scale diag(e^gamma) Q^ - P W   and   O_loc = P U~,
so that O = Q' H + O_loc.

The chunk grid restarts at every sequence start; the last chunk of a
sequence may be shorter than ``chunk``.  With chunk = 1 the evaluator is the
token recurrence itself.  Every exponent above is <= 0 when g <= 0.

Equality with the token recurrence for many chunk sizes is a pin
(``test_chunk_size_invariance`` and ``test_chunk_invariance_strong_decay``
in tests/test_oracle_invariants.py).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
from scipy.linalg import solve_triangular


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    return np.asarray(x, dtype=np.float64)


def _unit(x, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def chunk_step(Qh, Kh, V, g, b, H, scale=1.0):
    """One chunk from normalised rows.  Returns (intermediates dict, H')."""
    n = Kh.shape[0]
    gam = np.cumsum(g)
    diff = gam[:, None] - gam[None, :]
    causal = np.tril(np.ones((n, n), dtype=bool))
    D = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    G = Kh @ Kh.T
    A = np.tril(b[:, None] * D * G, k=-1)
    T = solve_triangular(np.eye(n) + A, np.eye(n), lower=True,
                         unit_diagonal=True)
    eg = np.exp(gam)
    W = T @ ((b * eg)[:, None] * Kh)
    Ut = T @ (b[:, None] * V)
    U = Ut - W @ H
    P = scale * D * (Qh @ Kh.T)
    O = scale * eg[:, None] * (Qh @ H) + P @ U
    Kt = np.exp(gam[-1] - gam)[:, None] * Kh
    Hn = np.exp(gam[-1]) * H + Kt.T @ U
    Qp = scale * eg[:, None] * Qh - P @ W
    inter = dict(gamma=gam, G=G, A=A, T=T, W=W, Utilde=Ut, U=U, P=P, O=O,
                 Ktilde=Kt, H_in=H.copy(), Qprime=Qp, Oloc=P @ Ut)
    return inter, Hn


def chunked_reference(q, k, v, g, beta, lengths: Sequence[int], init_state=None,
                      chunk: int = 64, scale: float = 1.0, eps: float = 1e-6,
                      keep: Optional[list] = None):
    """Chunked float64 evaluation over packed sequences.

    Same argument layout as ``oracle.reference``.  If ``keep`` is a list, one
    dict per (sequence, value head, chunk) is appended to it with keys
    seq, head, chunk, t0, n plus the intermediates of ``chunk_step``.
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    init = _f64(init_state)
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    grp = hv // hk
    out = np.zeros((T, hv, dv))
    final = np.zeros((len(lengths), hv, dk, dv))
    qn = _unit(q, eps)
    kn = _unit(k, eps)
    start = 0
    for i, L in enumerate(lengths):
        for h in range(hv):
            kh = h // grp
            H = np.zeros((dk, dv)) if init is None else init[i, h].copy()
            for c, t0 in enumerate(range(start, start + L, chunk)):
                t1 = min(t0 + chunk, start + L)
                inter, H = chunk_step(qn[t0:t1, kh], kn[t0:t1, kh],
                                      v[t0:t1, h], g[t0:t1, h],
                                      beta[t0:t1, h], H, scale)
                out[t0:t1, h] = inter["O"]
                if keep is not None:
                    inter.update(seq=i, head=h, chunk=c, t0=t0, n=t1 - t0)
                    keep.append(inter)
            final[i, h] = H
        start += L
    return out, final
