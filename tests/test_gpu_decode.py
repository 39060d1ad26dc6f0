"""Single-token decode step (GPU) against the float64 oracle.

gdn_decode applies one step of the recurrence to a state carried in memory.
The oracle computes exactly that when every sequence has length 1 and the
state is its initial state, so parity is checked against
oracle.reference(lengths=[1] * N, init_state=state).  A consistency case
checks that T decode steps on the GPU reproduce the GPU prefill of the same
T tokens.
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


def decode_inputs(name, n, **kw):
    kw.setdefault("init_std", 0.5)
    w = W.make_workload(name, lengths=[1] * n, **kw)
    dev = {x: getattr(w, x).cuda() for x in ("q", "k", "v", "g", "beta")}
    dev["state"] = w.init_state.clone().cuda()
    return w, dev


CASES = [
    ("bf16-16heads-d128", "prompt_4k", 4, dict(hk=16, hv=16, dk=128, dv=128)),
    ("bf16-gqa", "long_16k_gqa", 9, dict(hk=2, hv=6, dk=128, dv=64)),
    ("bf16-small", "prompt_4k", 255, dict(hk=1, hv=2, dk=16, dv=128)),
    ("bf16-dv16", "prompt_4k", 3, dict(hk=2, hv=2, dk=32, dv=16)),
    ("f32-d64", "tiny_fp32", 5, dict(hk=2, hv=4, dk=64, dv=32)),
    ("f32-d128", "tiny_fp32", 2, dict(hk=1, hv=1, dk=128, dv=128)),
    ("edge-beta0", "edge_mix", 6, dict(hk=1, hv=2, dk=64, dv=64, beta="zero")),
    ("edge-beta1-g0", "edge_mix", 6, dict(hk=1, hv=2, dk=64, dv=64, beta="one", g_low=0.0)),
]


@pytest.mark.parametrize("label,name,n,kw", CASES, ids=[c[0] for c in CASES])
def test_decode_matches_oracle(label, name, n, kw):
    w, d = decode_inputs(name, n, **kw)
    U.say(f"  decode {label}: N={n} {kw} dtype={w.q.dtype}")
    out = G.gdn_decode(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"],
                       opts=G.options(scale=0.75))
    torch.cuda.synchronize()
    ro, rf = oracle.reference(w.q, w.k, w.v, w.g, w.beta, w.lengths, w.init_state, scale=0.75)
    got_o = out.float().cpu().numpy()
    got_s = d["state"].cpu().numpy()
    es = U.rel_l2(got_s, rf)
    if w.q.dtype == torch.bfloat16:
        eo = U.max_abs(got_o, ro)
        U.say(f"    out max-abs {eo:.3e} (bf16 output), state rel-L2 {es:.3e}")
        # the arithmetic is fp32; only the stored output is rounded to bf16
        assert eo <= 2e-2 and eo <= 8e-3 * max(1.0, float(np.abs(ro).max()))
    else:
        eo = U.rel_l2(got_o, ro)
        U.say(f"    out rel-L2 {eo:.3e}, state rel-L2 {es:.3e}")
        assert eo <= U.F32_RELL2
    assert es <= U.F32_RELL2


def test_decode_zero_sequences_is_a_no_op():
    w, d = decode_inputs("prompt_4k", 1, hk=1, hv=1, dk=16, dv=16)
    e = {x: v[:0] for x, v in d.items()}
    out = G.gdn_decode(e["q"], e["k"], e["v"], e["g"], e["beta"], e["state"])
    torch.cuda.synchronize()
    assert out.shape[0] == 0


def test_decode_steps_reproduce_prefill():
    """T single-token steps from init give the prefill's outputs and state."""
    T = 40
    w = W.make_workload("long_16k_gqa", lengths=[T], hk=1, hv=3, dk=64, dv=64)
    dev = W.to_device(w)
    G.gdn_prefill_ex(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], None,
                     dev["init_state"], dev["out"], dev["final_state"])
    state = w.init_state.clone().cuda()
    outs = []
    for t in range(T):
        sl = slice(t, t + 1)
        outs.append(G.gdn_decode(dev["q"][sl], dev["k"][sl], dev["v"][sl], dev["g"][sl],
                                 dev["beta"][sl], state))
    torch.cuda.synchronize()
    dec_out = torch.cat(outs).float().cpu().numpy()
    ro, rf = oracle.reference(w.q, w.k, w.v, w.g, w.beta, w.lengths, w.init_state)
    U.say(f"  decode x{T}: out max-abs vs oracle {U.max_abs(dec_out, ro):.3e}; "
          f"prefill {U.max_abs(dev['out'].float().cpu().numpy(), ro):.3e}")
    # the decode path is fp32 throughout: tighter than the prefill's bf16 bound
    assert U.max_abs(dec_out, ro) <= 1e-2
    assert U.rel_l2(state.cpu().numpy(), rf) <= 1e-5
    # and the two GPU paths agree within the prefill's tolerances
    U.check_bf16(dev["out"].float().cpu().numpy(), dev["final_state"].cpu().numpy(),
                 dec_out, state.cpu().numpy(), "prefill vs decode")
