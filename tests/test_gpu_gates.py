"""The write gate given as raw projections (GDN_FLAG_BETA_LOGITS): the
kernels take beta = sigmoid(b) as they load it (GPU).

The inputs here are the workloads' own beta, turned back into logits
b = log(beta) - log(1 - beta) in float64 (so beta = 0 and 1 become -inf and
+inf); the oracle runs on beta itself.  Prefill and decode are checked
against the oracle, and beside the same call given beta directly (the two
differ only by the fp32 sigmoid's rounding).
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


def logits(beta: torch.Tensor) -> torch.Tensor:
    b = beta.double().numpy()
    with np.errstate(divide="ignore"):
        z = np.log(b) - np.log1p(-b)
    return torch.from_numpy(z.astype(np.float32))


CASES = [
    ("prompt_4k", dict(lengths=[700], hk=2, hv=2)),
    ("edge_mix", dict(hk=2, hv=2)),                      # beta ~0, ~1, sigmoid(N(0, 3)); ragged
    ("long_16k_gqa", dict(lengths=[300], hk=1, hv=3)),
    ("prompt_4k", dict(lengths=[64], hk=1, hv=1, beta="zero")),   # b = -inf everywhere
    ("prompt_4k", dict(lengths=[64], hk=1, hv=1, beta="one")),    # b = +inf everywhere
]


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_prefill_beta_logits(name, kw):
    w = W.make_workload(name, **kw)
    ro, rf = oracle.reference_workload(w)
    d = W.to_device(w)
    cu = d["cu_seqlens"] if w.n_seqs > 1 else None
    z = logits(w.beta).cuda()
    U.say(f"  gpu run: {name} {kw}, beta as logits")
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], z, cu, d["init_state"], d["out"],
                     d["final_state"], opts=G.options(chunk=w.chunk, beta_logits=True))
    torch.cuda.synchronize()
    out_z, fin_z = d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy()
    U.check_bf16(out_z, fin_z, ro, rf, label=f"{name} logits")
    out_b, fin_b, _ = U.run_gpu(w)
    dz = U.max_abs(out_z, out_b)
    U.say(f"  logits vs beta: out max-abs {dz:.3e}, final rel-L2 {U.rel_l2(fin_z, fin_b):.3e}")


@pytest.mark.parametrize("name,n,kw", [("prompt_4k", 5, dict(hk=2, hv=2, dk=128, dv=128)),
                                       ("edge_mix", 7, dict(hk=1, hv=2, dk=64, dv=64)),
                                       ("tiny_fp32", 3, dict(hk=1, hv=2, dk=32, dv=32))])
def test_decode_beta_logits(name, n, kw):
    w = W.make_workload(name, lengths=[1] * n, init_std=0.5, **kw)
    ro, rf = oracle.reference(w.q, w.k, w.v, w.g, w.beta, w.lengths, w.init_state)
    dev = {x: getattr(w, x).cuda() for x in ("q", "k", "v", "g")}
    state = w.init_state.clone().cuda()
    U.say(f"  decode: {name} N={n} {kw}, beta as logits")
    out = G.gdn_decode(dev["q"], dev["k"], dev["v"], dev["g"], logits(w.beta).cuda(), state,
                       opts=G.options(beta_logits=True))
    torch.cuda.synchronize()
    es = U.rel_l2(state.cpu().numpy(), rf)
    eo = U.max_abs(out.float().cpu().numpy(), ro)
    U.say(f"    out max-abs {eo:.3e}, state rel-L2 {es:.3e}")
    if w.q.dtype == torch.bfloat16:
        assert eo <= U.BF16_OUT_MAXABS and es <= U.BF16_STATE_RELL2
    else:
        assert U.rel_l2(out.float().cpu().numpy(), ro) <= 1e-5 and es <= 1e-5
