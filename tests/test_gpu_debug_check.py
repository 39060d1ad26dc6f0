"""GDN_DEBUG_CHECK=1 (GPU): a packed prefill checks cu_seqlens on the device
before anything else is enqueued.

A malformed table (an entry below its predecessor; a first entry other than
0; a last entry past T) makes the call return GDN_ERR_INPUT, and the output
keeps its sentinel values because nothing after the check ran.  A
well-formed table passes the check and gives the oracle's result.  Without
the variable the same malformed table is only clamped (no error), as the
header documents.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()
    oracle.load()


BAD = {
    "decreasing": [0, 50, 40, 120],
    "first_nonzero": [3, 50, 90, 120],
    "past_end": [0, 50, 90, 121],
}


@pytest.mark.parametrize("dtype", [torch.int32, torch.int64], ids=["int32", "int64"])
@pytest.mark.parametrize("case", sorted(BAD))
def test_malformed_table_is_rejected(monkeypatch, case, dtype):
    monkeypatch.setenv("GDN_DEBUG_CHECK", "1")
    w = W.make_workload("packed_255", lengths=[50, 40, 30], hk=1, hv=2)
    d = W.to_device(w)
    cu = torch.tensor(BAD[case], dtype=dtype, device="cuda")
    out = torch.full_like(d["out"], 7.0)
    U.say(f"  debug check, {case}: cu = {BAD[case]}")
    with pytest.raises(G.GdnError) as ei:
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, None, out, None)
    torch.cuda.synchronize()
    assert ei.value.status == -8 and "GDN_DEBUG_CHECK" in str(ei.value)
    assert torch.all(out == 7.0)


def test_wellformed_table_passes(monkeypatch):
    monkeypatch.setenv("GDN_DEBUG_CHECK", "1")
    w = W.make_workload("packed_255", lengths=[50, 0, 40, 30], hk=1, hv=2)
    out, fin, _ = U.run_gpu(w)
    ro, rf = oracle.reference_workload(w)
    U.check_bf16(out, fin, ro, rf, label="debug check, well-formed table")


def test_without_the_check_a_bad_table_is_clamped(monkeypatch):
    monkeypatch.delenv("GDN_DEBUG_CHECK", raising=False)
    w = W.make_workload("packed_255", lengths=[50, 40, 30], hk=1, hv=2)
    d = W.to_device(w)
    cu = torch.tensor(BAD["decreasing"], dtype=torch.int32, device="cuda")
    out = torch.full_like(d["out"], 7.0)
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, None, out, None)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
