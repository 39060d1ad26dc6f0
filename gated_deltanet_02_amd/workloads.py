"""Seeded synthetic inputs for the chunked Gated DeltaNet prefill.

This module only draws random numbers and moves data; it holds none of the
method's arithmetic, so both the float64 oracle (under ``oracle/``) and the HIP
path can take their inputs from it without sharing any computation.

The workloads stand in for the prompts the pages serve: one prompt per
candidate, up to 4096 tokens by default and 16384 at most ("Open-Jev-27B-v1.1
native text worker", section "Prepare the checkpoint"), 1-255 candidates per
question (same page, introduction).  No dataset, prompt or weight is used.

Recipe (fixed draw order: lengths -> q -> k -> v -> g -> g-zero rows ->
beta -> init, numpy PCG64 seeded with ``seed``):

* q, k: rows drawn N(0, 1) in float32 and mapped onto the unit sphere (a
  Gaussian row divided by its Euclidean length is a uniform unit vector), then
  rounded to the storage dtype (bf16 round-to-nearest-even via torch);
* v: N(0, 1) float32, rounded to the storage dtype;
* g: the log-decay, U(g_low, 0) float32; optionally a drawn fraction of token
  rows is set to exactly 0 for all heads;
* beta: the already-activated write strength, sigmoid of N(0, 1), or for the
  edge mix one of three classes per (token, head): sigmoid(-12), sigmoid(12),
  sigmoid(N(0, 3)), each drawn with probability 1/3;
* init: zeros (passed as NULL) or N(0, init_std) float32.

The q and k rows may instead be left un-normalised, so that the library's
own L2 normalisation is what makes them unit rows (``qk_rows``):

* "unit" (default): as above;
* "raw": the same Gaussian rows, not divided by their length (norm about
  sqrt(d));
* "scaled": the unit rows, then (drawn after init, so the other draws are
  unchanged) each (token, key head) row of q and of k multiplied by a factor
  of one class: 0 (a zero row, 4 %), 1e-3 (squared norm 1e-6, the size of
  the default eps, 8 %), 1e3 (4 %), else log-uniform in [0.05, 20].

The gates on either side of the prefill (``make_gate_inputs``, drawn from
their own seeded stream so the workload above is unchanged): the decay
gate's raw projection a ~ N(0, 1) float32 per (token, value head); per value
head A = log U(1, 16) and bias ~ U(-6.9, -2.3) (so softplus(a + bias) spans
about 1e-4 .. 1 and the decay rate e^A 1 .. 16); the output gate's projection
z ~ N(0, 1) rounded to v's dtype; the norm weight 1 + 0.1 N(0, 1) float32.
``make_gate_rows`` draws standalone rows for the output gate alone: rows of
N(0, 1) times a per-row factor (0, 1e-3, 1e3 or log-uniform in [0.05, 20],
as "scaled" above), z ~ N(0, 2) with a few entries at +-30.

The short convolution before the activation (``make_conv_inputs``, its own
seeded stream): taps N(0, 1/W) float32 over the D = 2 Hk dk + Hv dv
channels (q | k | v), plus 1 on the last tap (so the current token keeps a
share of about one); history rows [N, W - 1, D] drawn as the inputs are
(unit q and k rows per key head, v N(0, 1)), rounded to the storage dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "SPECS",
    "Workload",
    "GateInputs",
    "make_gate_inputs",
    "make_gate_rows",
    "make_conv_inputs",
    "make_workload",
    "permute_sequences",
    "select_sequences",
    "select_key_head",
    "to_device",
]


# name -> shape/distribution recipe.  ``lengths`` is a list of per-sequence
# token counts, or ("uniform", n, lo, hi) for n lengths drawn from
# rng.integers(lo, hi + 1).
SPECS = {
    # batch 1, T=64, 2 heads, d=16, chunk 16, float32 inputs
    "tiny_fp32": dict(lengths=[64], hk=2, hv=2, dk=16, dv=16, chunk=16,
                      dtype="fp32", g_low=-0.5, beta="sigmoid_normal",
                      init_std=None, g_zero_frac=0.0, token_offset=0),
    # batch 1, T=4096, 16 heads, d=128, chunk 64, bf16 (the throughput workload)
    "prompt_4k": dict(lengths=[4096], hk=16, hv=16, dk=128, dv=128, chunk=64,
                      dtype="bf16", g_low=-1.0, beta="sigmoid_normal",
                      init_std=None, g_zero_frac=0.0, token_offset=0),
    # batch 1, T=16384, 16 q/k heads shared by 48 value heads, random init state
    "long_16k_gqa": dict(lengths=[16384], hk=16, hv=48, dk=128, dv=128,
                         chunk=64, dtype="bf16", g_low=-1.0,
                         beta="sigmoid_normal", init_std=0.1, g_zero_frac=0.0,
                         token_offset=0),
    # 255 independent prompts, lengths U[200, 4096], packed via cu_seqlens
    "packed_255": dict(lengths=("uniform", 255, 200, 4096), hk=16, hv=16,
                       dk=128, dv=128, chunk=64, dtype="bf16", g_low=-1.0,
                       beta="sigmoid_normal", init_std=None, g_zero_frac=0.0,
                       token_offset=0),
    # numerics edge set: ragged lengths, strong decay mixed with g=0 rows,
    # beta near 0 / near 1 / wide sigmoid, q/k/v one token into their storage
    "edge_mix": dict(lengths=[1, 63, 64, 65, 1000], hk=8, hv=8, dk=128,
                     dv=128, chunk=64, dtype="bf16", g_low=-8.0,
                     beta="three_class", init_std=None, g_zero_frac=0.25,
                     token_offset=1),
    # decode: one token for each of 256 sequences, 16 heads, d=128, bf16,
    # against a carried fp32 state (the step after a prefill)
    "decode_256": dict(lengths=[1] * 256, hk=16, hv=16, dk=128, dv=128,
                       chunk=64, dtype="bf16", g_low=-1.0, beta="sigmoid_normal",
                       init_std=0.5, g_zero_frac=0.0, token_offset=0),
}

# Row factor classes of qk_rows="scaled": (probability, factor); None is
# the log-uniform class.
SCALED_ROW_CLASSES = ((0.04, 0.0), (0.08, 1e-3), (0.04, 1e3), (0.84, None))
SCALED_ROW_RANGE = (0.05, 20.0)


@dataclasses.dataclass
class Workload:
    """Host-side inputs of one prefill call (CPU tensors)."""

    name: str
    q: torch.Tensor            # [T, Hk, dk]  bf16 or fp32
    k: torch.Tensor            # [T, Hk, dk]
    v: torch.Tensor            # [T, Hv, dv]
    g: torch.Tensor            # [T, Hv] fp32 log-decay (<= 0)
    beta: torch.Tensor         # [T, Hv] fp32 in [0, 1]
    lengths: list              # per-sequence token counts
    init_state: Optional[torch.Tensor]  # [N, Hv, dk, dv] fp32 or None
    chunk: int
    token_offset: int          # storage offset (tokens) of q/k/v on device

    @property
    def n_seqs(self) -> int:
        return len(self.lengths)

    @property
    def t_total(self) -> int:
        return int(self.q.shape[0])

    @property
    def cu_seqlens(self) -> torch.Tensor:
        cu = np.zeros(len(self.lengths) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(np.asarray(self.lengths, dtype=np.int64))
        return torch.from_numpy(cu.astype(np.int32))

    @property
    def dims(self):
        return dict(T=self.t_total, N=self.n_seqs, hk=self.q.shape[1],
                    hv=self.v.shape[1], dk=self.q.shape[2], dv=self.v.shape[2])


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _unit_rows(rng, shape) -> np.ndarray:
    """Rows drawn uniformly on the unit sphere (float32)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    n = np.sqrt(np.sum(x.astype(np.float64) ** 2, axis=-1, keepdims=True))
    n[n == 0] = 1.0
    return (x / n).astype(np.float32)


def _gauss_rows(rng, shape) -> np.ndarray:
    """The same draws as ``_unit_rows``, left un-normalised."""
    return rng.standard_normal(shape, dtype=np.float32)


def _row_factors(rng, shape) -> np.ndarray:
    """One factor per row from SCALED_ROW_CLASSES (float32)."""
    u = rng.random(shape)
    lo, hi = SCALED_ROW_RANGE
    f = np.exp(rng.uniform(np.log(lo), np.log(hi), size=shape))
    edge = 0.0
    for p, val in SCALED_ROW_CLASSES:
        if val is None:
            continue
        f = np.where((u >= edge) & (u < edge + p), val, f)
        edge += p
    return f.astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype == "bf16":
        return t.to(torch.bfloat16)  # round-to-nearest-even
    if dtype == "fp32":
        return t.to(torch.float32)
    raise ValueError(dtype)


def make_workload(name: str, seed: int = 0, **overrides) -> Workload:
    """Draw the named workload; ``overrides`` replace recipe fields
    (e.g. ``lengths=[300]`` or ``hv=4``) to make reduced test cases."""
    spec = dict(SPECS[name])
    spec.update(overrides)
    rng = np.random.default_rng(seed)
    lens = spec["lengths"]
    if isinstance(lens, tuple) and lens[0] == "uniform":
        _, n, lo, hi = lens
        lengths = [int(x) for x in rng.integers(lo, hi + 1, size=n)]
    else:
        lengths = [int(x) for x in lens]
    T = int(sum(lengths))
    hk, hv, dk, dv = spec["hk"], spec["hv"], spec["dk"], spec["dv"]
    if hv % hk:
        raise ValueError("hv must be a multiple of hk")
    qk_rows = spec.get("qk_rows", "unit")
    if qk_rows not in ("unit", "raw", "scaled"):
        raise ValueError(qk_rows)
    rows = _gauss_rows if qk_rows == "raw" else _unit_rows
    q = rows(rng, (T, hk, dk))
    k = rows(rng, (T, hk, dk))
    v = rng.standard_normal((T, hv, dv), dtype=np.float32)
    g = rng.uniform(spec["g_low"], 0.0, size=(T, hv)).astype(np.float32)
    if spec["g_zero_frac"] > 0:
        nz = int(round(spec["g_zero_frac"] * T))
        rows = rng.choice(T, size=nz, replace=False)
        g[rows, :] = 0.0
    if spec["beta"] == "sigmoid_normal":
        beta = _sigmoid(rng.standard_normal((T, hv)))
    elif spec["beta"] == "three_class":
        cls = rng.integers(0, 3, size=(T, hv))
        wide = _sigmoid(3.0 * rng.standard_normal((T, hv)))
        beta = np.where(cls == 0, _sigmoid(np.float32(-12.0)),
                        np.where(cls == 1, _sigmoid(np.float32(12.0)), wide))
        beta = beta.astype(np.float32)
    elif spec["beta"] == "zero":
        beta = np.zeros((T, hv), np.float32)
    elif spec["beta"] == "one":
        beta = np.ones((T, hv), np.float32)
    else:
        raise ValueError(spec["beta"])
    init = None
    if spec["init_std"] is not None:
        init = torch.from_numpy(
            (spec["init_std"] * rng.standard_normal(
                (len(lengths), hv, dk, dv), dtype=np.float32)).astype(np.float32))
    if qk_rows == "scaled":
        q = q * _row_factors(rng, (T, hk))[..., None]
        k = k * _row_factors(rng, (T, hk))[..., None]
    dt = spec["dtype"]
    return Workload(name=name, q=_store(q, dt), k=_store(k, dt),
                    v=_store(v, dt), g=torch.from_numpy(g),
                    beta=torch.from_numpy(beta), lengths=lengths,
                    init_state=init, chunk=int(spec["chunk"]),
                    token_offset=int(spec["token_offset"]))


def _seq_rows(w: Workload, i: int) -> slice:
    start = int(sum(w.lengths[:i]))
    return slice(start, start + w.lengths[i])


def permute_sequences(w: Workload, order: Sequence[int]) -> Workload:
    """Repack the same sequences in another order (pure data movement)."""
    parts = [_seq_rows(w, i) for i in order]
    cat = lambda t: torch.cat([t[s] for s in parts], 0)  # noqa: E731
    init = None if w.init_state is None else w.init_state[list(order)].clone()
    return dataclasses.replace(
        w, name=w.name + "_perm", q=cat(w.q), k=cat(w.k), v=cat(w.v),
        g=cat(w.g), beta=cat(w.beta),
        lengths=[w.lengths[i] for i in order], init_state=init)


def select_sequences(w: Workload, idx: Sequence[int]) -> Workload:
    """A workload made of a subset of the sequences (pure data movement)."""
    return permute_sequences(w, list(idx))


def select_key_head(w: Workload, kh: int) -> Workload:
    """Keep key head ``kh`` and the value heads that read it
    (value head h reads key head h // (Hv/Hk))."""
    hk, hv = w.q.shape[1], w.v.shape[1]
    grp = hv // hk
    vs = slice(kh * grp, (kh + 1) * grp)
    init = None if w.init_state is None else w.init_state[:, vs].contiguous()
    return dataclasses.replace(
        w, q=w.q[:, kh:kh + 1].contiguous(), k=w.k[:, kh:kh + 1].contiguous(),
        v=w.v[:, vs].contiguous(), g=w.g[:, vs].contiguous(),
        beta=w.beta[:, vs].contiguous(), init_state=init)


def _offset_view(x: torch.Tensor, off: int, device) -> torch.Tensor:
    """Copy ``x`` to ``device`` as a view starting ``off`` tokens into a
    larger allocation (a non-zero storage offset)."""
    if off == 0:
        return x.to(device).contiguous()
    buf = torch.zeros((x.shape[0] + 2 * off,) + tuple(x.shape[1:]),
                      dtype=x.dtype, device=device)
    view = buf[off:off + x.shape[0]]
    view.copy_(x.to(device))
    return view


def to_device(w: Workload, device="cuda"):
    """Device copies of the inputs plus freshly allocated outputs."""
    q = _offset_view(w.q, w.token_offset, device)
    k = _offset_view(w.k, w.token_offset, device)
    v = _offset_view(w.v, w.token_offset, device)
    g = w.g.to(device).contiguous()
    beta = w.beta.to(device).contiguous()
    cu = w.cu_seqlens.to(device)
    init = None if w.init_state is None else w.init_state.to(device).contiguous()
    out = torch.empty(w.v.shape, dtype=w.v.dtype, device=device)
    final = torch.empty((w.n_seqs, w.v.shape[1], w.q.shape[2], w.v.shape[2]),
                        dtype=torch.float32, device=device)
    return dict(q=q, k=k, v=v, g=g, beta=beta, cu_seqlens=cu,
                init_state=init, out=out, final_state=final)


@dataclasses.dataclass
class GateInputs:
    a: torch.Tensor        # [T, Hv] fp32: the decay gate's raw projection
    a_log: torch.Tensor    # [Hv] fp32: log of the per-head decay rate
    bias: torch.Tensor     # [Hv] fp32: per-head shift of the projection
    z: torch.Tensor        # [T, Hv, dv] in v's dtype: the output gate's projection
    norm_w: torch.Tensor   # [dv] fp32: the output norm's weight


def make_gate_inputs(w: Workload, seed: int = 1) -> GateInputs:
    """Seeded gate inputs shaped for workload ``w`` (recipe in the module
    docstring; fixed draw order a -> A -> bias -> z -> weight)."""
    rng = np.random.default_rng([seed, 0x6A7E])
    T, hv, dv = w.v.shape
    a = rng.standard_normal((T, hv), dtype=np.float32)
    a_log = np.log(rng.uniform(1.0, 16.0, size=hv)).astype(np.float32)
    bias = rng.uniform(-6.9, -2.3, size=hv).astype(np.float32)
    z = rng.standard_normal((T, hv, dv), dtype=np.float32)
    nw = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    dt = "bf16" if w.v.dtype == torch.bfloat16 else "fp32"
    return GateInputs(a=torch.from_numpy(a), a_log=torch.from_numpy(a_log),
                      bias=torch.from_numpy(bias), z=_store(z, dt), norm_w=torch.from_numpy(nw))


def make_gate_rows(rows: int, heads: int, dv: int, dtype: str = "bf16", seed: int = 2):
    """Standalone rows for the output gate: x, z [rows, heads, dv] in
    ``dtype``, weight [dv] fp32 (recipe in the module docstring)."""
    rng = np.random.default_rng([seed, 0x6A7F])
    x = rng.standard_normal((rows, heads, dv), dtype=np.float32)
    x *= _row_factors(rng, (rows, heads))[..., None]
    z = 2.0 * rng.standard_normal((rows, heads, dv), dtype=np.float32)
    hot = rng.random((rows, heads, dv)) < 0.01
    z = np.where(hot, np.where(rng.random((rows, heads, dv)) < 0.5, 30.0, -30.0), z).astype(np.float32)
    nw = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    return _store(x, dtype), _store(z, dtype), torch.from_numpy(nw)


def make_conv_inputs(w: Workload, width: int = 4, seed: int = 3):
    """Taps [D, W] fp32 and history rows [N, W - 1, D] in the workload's
    dtype for the short convolution (recipe in the module docstring; draw
    order taps -> q history -> k history -> v history)."""
    rng = np.random.default_rng([seed, 0xC0DE])
    T, hk, dk = w.q.shape
    hv, dv = w.v.shape[1], w.v.shape[2]
    D = 2 * hk * dk + hv * dv
    taps = rng.standard_normal((D, width), dtype=np.float32) / np.float32(np.sqrt(width))
    taps[:, width - 1] += 1.0
    n, h = w.n_seqs, width - 1
    hq = _unit_rows(rng, (n, h, hk, dk)).reshape(n, h, hk * dk)
    hkk = _unit_rows(rng, (n, h, hk, dk)).reshape(n, h, hk * dk)
    hvv = rng.standard_normal((n, h, hv * dv), dtype=np.float32)
    dt = "bf16" if w.q.dtype == torch.bfloat16 else "fp32"
    hist = np.concatenate([hq, hkk, hvv], axis=2).astype(np.float32)
    return torch.from_numpy(taps.astype(np.float32)), _store(hist, dt)
