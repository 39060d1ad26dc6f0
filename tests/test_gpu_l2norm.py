"""The fused L2 normalisation of q and k on the GPU, against the oracle.

The library divides each q and k row by sqrt(|x|^2 + eps) before use; the
oracle does the same in float64.  The ordinary workloads already have unit
rows, which hides that step, so these cases draw rows that are not unit
rows: "raw" Gaussian rows (norm about sqrt(d)) and "scaled" rows (unit rows
times a per-row factor: zero rows, rows with |x|^2 = 1e-6 = eps, rows of
norm 1e3, and log-uniform factors in [0.05, 20]).  Each output is compared
element by element with the oracle at the stated bounds: bf16 inputs
max-abs 2e-2 on outputs and rel-L2 5e-3 on the state, fp32 inputs rel-L2
1e-5.

What a kernel that skipped the normalisation would show on these inputs
(float64 chunked evaluator with the normalisation removed, computed in
tests/test_l2norm_sensitivity.py, which requires at least five times the
bf16 bounds):
raw rows, 377 tokens: outputs off by ~2e+104 (|1 - beta |k|^2| ~ 60 per
token); scaled rows, 377 tokens: ~1.5e+26; scaled edge mix: ~6.8e+7;
scaled fp32, d=16: ~7e+28.  Using eps = 1e-6 where 1e-2 was asked moves
the scaled outputs by 0.31 (state rel-L2 0.42).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import oracle
from tests import gpu_util as U

# (id, workload, overrides); every chunk size of each dtype is run
PREFILL_CASES = [
    ("bf16-raw", "prompt_4k", dict(lengths=[300, 77], hk=2, hv=4, qk_rows="raw")),
    ("bf16-scaled", "prompt_4k", dict(lengths=[300, 77], hk=2, hv=4, qk_rows="scaled")),
    ("bf16-scaled-gqa-d64", "long_16k_gqa", dict(lengths=[190], hk=2, hv=6, dk=64, dv=64,
                                                 qk_rows="scaled")),
    ("bf16-edge-scaled", "edge_mix", dict(hk=2, hv=2, qk_rows="scaled")),
    ("f32-raw", "tiny_fp32", dict(qk_rows="raw")),
    ("f32-scaled", "tiny_fp32", dict(qk_rows="scaled")),
    ("f32-scaled-d128", "tiny_fp32", dict(lengths=[200, 33], hk=1, hv=2, dk=128, dv=128,
                                          chunk=32, qk_rows="scaled")),
]
BF16_CHUNKS = (64, 32, 16)
F32_CHUNKS = (32, 16)
# a non-default eps, on rows whose |x|^2 is near it
EPS_CASE = ("prompt_4k", dict(lengths=[300, 77], hk=2, hv=4, qk_rows="scaled"), 1e-2)


def _prefill_params():
    out = []
    for label, name, kw in PREFILL_CASES:
        chunks = F32_CHUNKS if name == "tiny_fp32" else BF16_CHUNKS
        for c in chunks:
            if name == "tiny_fp32" and kw.get("dk", 16) == 128 and c == 64:
                continue
            out.append(pytest.param(label, name, kw, c, id=f"{label}-c{c}", marks=pytest.mark.gpu))
    return out


def _check(w, out, fin, ro, rf, label):
    if w.q.dtype == torch.bfloat16:
        U.check_bf16(out, fin, ro, rf, label=label)
    else:
        U.check_f32(out, fin, ro, rf, label=label)


@pytest.mark.parametrize("label,name,kw,chunk", _prefill_params())
def test_prefill_nonunit_rows(label, name, kw, chunk):
    U.need_gpu()
    w = W.make_workload(name, **kw)
    out, fin, _ = U.run_gpu(w, chunk=chunk)
    ro, rf = oracle.reference_workload(w)
    _check(w, out, fin, ro, rf, f"{label} chunk {chunk}")


@pytest.mark.gpu
@pytest.mark.parametrize("chunk", BF16_CHUNKS)
def test_prefill_non_default_eps(chunk):
    U.need_gpu()
    name, kw, eps = EPS_CASE
    w = W.make_workload(name, **kw)
    d = W.to_device(w)
    U.say(f"  eps {eps} chunk {chunk}")
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], None,
                     d["out"], d["final_state"], opts=G.options(chunk=chunk, l2_eps=eps))
    torch.cuda.synchronize()
    ro, rf = oracle.reference_workload(w, eps=eps)
    U.check_bf16(d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf,
                 label=f"eps {eps} chunk {chunk}")


@pytest.mark.gpu
def test_prompt_4k_full_raw_rows():
    """The benchmark shape (T=4096, 16 heads, d=128, bf16) with raw Gaussian
    q/k rows: every output and the whole state against the oracle."""
    U.need_gpu()
    w = W.make_workload("prompt_4k", qk_rows="raw")
    out, fin, _ = U.run_gpu(w)
    ro, rf = oracle.reference_workload(w)
    U.check_bf16(out, fin, ro, rf, label="prompt_4k raw rows")


DECODE_CASES = [
    ("bf16-scaled", "prompt_4k", 64, dict(hk=4, hv=8, dk=128, dv=128, qk_rows="scaled"), 1e-6),
    ("bf16-raw", "prompt_4k", 16, dict(hk=2, hv=2, dk=64, dv=128, qk_rows="raw"), 1e-6),
    ("bf16-scaled-eps", "prompt_4k", 64, dict(hk=4, hv=8, dk=128, dv=128, qk_rows="scaled"), 1e-2),
    ("f32-scaled", "tiny_fp32", 64, dict(hk=2, hv=4, dk=64, dv=32, qk_rows="scaled"), 1e-6),
]


@pytest.mark.gpu
@pytest.mark.parametrize("label,name,n,kw,eps", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_nonunit_rows(label, name, n, kw, eps):
    U.need_gpu()
    w = W.make_workload(name, lengths=[1] * n, init_std=0.5, **kw)
    dev = {x: getattr(w, x).cuda() for x in ("q", "k", "v", "g", "beta")}
    state = w.init_state.clone().cuda()
    U.say(f"  decode {label}: N={n} eps={eps}")
    out = G.gdn_decode(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state,
                       opts=G.options(l2_eps=eps))
    torch.cuda.synchronize()
    ro, rf = oracle.reference(w.q, w.k, w.v, w.g, w.beta, w.lengths, w.init_state, eps=eps)
    got_o, got_s = out.float().cpu().numpy(), state.cpu().numpy()
    es = U.rel_l2(got_s, rf)
    if w.q.dtype == torch.bfloat16:
        eo = U.max_abs(got_o, ro)
        U.say(f"    out max-abs {eo:.3e}, state rel-L2 {es:.3e}")
        assert eo <= 2e-2 and eo <= 8e-3 * max(1.0, float(np.abs(ro).max()))
    else:
        eo = U.rel_l2(got_o, ro)
        U.say(f"    out rel-L2 {eo:.3e}, state rel-L2 {es:.3e}")
        assert eo <= U.F32_RELL2
    assert es <= U.F32_RELL2
