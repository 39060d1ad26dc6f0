"""The GPU L2-norm cases can see the normalisation (CPU).

The q and k rows of the ordinary workloads are unit rows, so a kernel that
skipped the L2 normalisation, or applied eps wrongly, would stay inside the
parity tolerances on them.  The cases of tests/test_gpu_l2norm.py use rows
that are not unit rows (``qk_rows`` "raw" and "scaled" in the input module)
and a non-default eps.  These checks plant each such mistake in the float64
chunked evaluator and require that the result moves far beyond the GPU
tolerances (2e-2 max-abs on outputs, 5e-3 rel-L2 on the state for bf16;
1e-5 rel-L2 for fp32), so that the GPU cases would catch the same mistake
in a kernel.
"""
import warnings

import numpy as np
import pytest

from gated_deltanet_02_amd import workloads as W
from oracle import chunked, oracle

from tests.test_gpu_l2norm import PREFILL_CASES, EPS_CASE


def _with_unit(fn, w, chunk, eps):
    orig = chunked._unit
    chunked._unit = fn
    try:
        with warnings.catch_warnings(), np.errstate(all="ignore"):
            warnings.simplefilter("ignore")
            return chunked.chunked_reference(w.q, w.k, w.v, w.g, w.beta, w.lengths,
                                             w.init_state, chunk=chunk, eps=eps)
    finally:
        chunked._unit = orig


def _errors(o, f, ro, rf):
    with np.errstate(all="ignore"):
        if not (np.isfinite(o).all() and np.isfinite(f).all()):
            return np.inf, np.inf
        return float(np.abs(o - ro).max()), float(np.linalg.norm(f - rf) / np.linalg.norm(rf))


MUTANTS = {
    "no normalisation": lambda x, eps: x,
    "eps outside the root": lambda x, eps: x / (np.sqrt(np.sum(x * x, -1, keepdims=True)) + eps),
    "eps ignored": lambda x, eps: x / np.sqrt(np.sum(x * x, -1, keepdims=True) + 1e-30),
}


@pytest.mark.parametrize("label,name,kw", [(c[0], c[1], c[2]) for c in PREFILL_CASES],
                         ids=[c[0] for c in PREFILL_CASES])
def test_mistakes_are_visible(label, name, kw):
    w = W.make_workload(name, **kw)
    ro, rf = oracle.reference_workload(w)
    for mname, fn in MUTANTS.items():
        if mname != "no normalisation" and kw.get("qk_rows") == "raw":
            continue  # raw rows have |x|^2 ~ d: eps mistakes are invisible there by design
        if mname == "eps ignored" and not np.any(w.k.float().norm(dim=-1).numpy() == 0):
            continue
        o, f = _with_unit(fn, w, 16, 1e-6)
        ea, es = _errors(o, f, ro, rf)
        # at least five times the looser (bf16) bounds
        assert ea > 0.1 or es > 0.025, f"{label}: '{mname}' moves out by {ea}, state by {es}"


def test_non_default_eps_is_visible():
    name, kw, eps = EPS_CASE
    w = W.make_workload(name, **kw)
    ro, rf = oracle.reference_workload(w, eps=eps)
    r0, f0 = oracle.reference_workload(w)
    ea, es = _errors(r0, f0, ro, rf)
    assert ea > 0.2 and es > 0.05, (ea, es)
