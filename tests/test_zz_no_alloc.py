"""gdn_prefill_noalloc (the prefill on the library's static device scratch)
against gdn_prefill_ex on the same inputs, through the C ABI (GPU).

Both entry points launch the same kernels in the same order, so their outputs
and final states must be bitwise equal.  Two calls in a row, the second with
a smaller input, show that the scratch's leftover contents from the first
call do not leak into the second; a call whose workspace would exceed the
scratch is rejected before anything runs.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


def _both(w, opts=None):
    """(noalloc out, final), (ex out, final) on fresh device copies."""
    res = []
    for entry in ("noalloc", "ex"):
        d = W.to_device(w)
        cu = d["cu_seqlens"] if w.n_seqs > 1 else None
        d["out"].fill_(3.0)
        d["final_state"].fill_(3.0)
        U.say(f"  {entry}: {w.name} T={w.t_total} N={w.n_seqs} Hv={w.v.shape[1]}")
        if entry == "noalloc":
            G.gdn_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"],
                                  d["out"], d["final_state"], opts=opts)
        else:
            G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"],
                             d["out"], d["final_state"], opts=opts)
        torch.cuda.synchronize()
        res.append((d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy()))
    return res


def test_noalloc_matches_ex_two_calls():
    U.need_gpu()
    big = W.make_workload("prompt_4k")                       # 64 MiB of workspace
    small = W.make_workload("edge_mix", hk=2, hv=2)          # packed, ragged, far smaller
    lay_big = G.gdn_workspace_size(*[W.to_device(big)[x] for x in ("q", "k", "v")])
    assert lay_big <= G.NOALLOC_SCRATCH_BYTES
    for w in (big, small):
        (no, nf), (eo, ef) = _both(w)
        assert np.array_equal(no, eo), f"{w.name}: outputs differ"
        assert np.array_equal(nf, ef), f"{w.name}: final states differ"
    # and the smaller call is right on its own terms
    ro, rf = oracle.reference_workload(small)
    U.check_bf16(no, nf, ro, rf, label="noalloc edge_mix")


def test_noalloc_rejects_oversize():
    U.need_gpu()
    w = W.make_workload("prompt_4k", lengths=[8192], hk=1, hv=1, dk=16, dv=16)
    d = W.to_device(w)
    need = G.gdn_workspace_size(d["q"], d["k"], d["v"])
    assert need <= G.NOALLOC_SCRATCH_BYTES
    big = W.make_workload("prompt_4k", lengths=[7000], hk=16, hv=16)
    d = W.to_device(big)
    need = G.gdn_workspace_size(d["q"], d["k"], d["v"])
    assert need > G.NOALLOC_SCRATCH_BYTES
    with pytest.raises(G.GdnError) as ei:
        G.gdn_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None,
                              d["out"], d["final_state"])
    assert ei.value.status == -6  # GDN_ERR_WORKSPACE
