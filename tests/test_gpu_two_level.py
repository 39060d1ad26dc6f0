"""The two-level scan (scan_split = SCAN_TWO_LEVEL) against the float64
oracle (GPU), beside the one-pass scan on the same inputs.

The two-level scan splits each sequence (at about 17/32 of its chunks), scans the
second part from zero beside the product of its chunk transitions, and
corrects the second part's outputs and the final state; the oracle is the
token recurrence, which knows nothing of segments.  Cases cover an odd
number of chunks with a partial last one, grouped value heads with a
random initial state, chunks of 32, the smallest split (two chunks), a
uniform batch given as 4-D tensors, no final state, and the full
4096-token prompt.
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


CASES = [
    ("prompt_4k", dict(lengths=[1000], hk=4, hv=4)),                      # 16 chunks, partial last
    ("prompt_4k", dict(lengths=[333], hk=2, hv=2, dk=64, dv=64)),         # 6 chunks
    ("long_16k_gqa", dict(lengths=[700], hk=2, hv=6)),                    # groups of 3, init state
    ("prompt_4k", dict(lengths=[190], hk=2, hv=4, dk=128, dv=64, chunk=32)),
    ("prompt_4k", dict(lengths=[100], hk=1, hv=2)),                       # 2 chunks: split 1 + 1
    ("edge_mix", dict(lengths=[1000], hk=2, hv=2)),                       # strong decay, g = 0 rows
    ("long_16k_gqa", dict(lengths=[400], hk=8, hv=16)),                   # 8 key heads: permuted head order
    # weak decay: the state at the split reaches every later chunk, so the
    # transition product (not only its first, identity, factor) decides the
    # second half
    ("prompt_4k", dict(lengths=[2048], hk=2, hv=2, g_low=-0.02)),
    ("long_16k_gqa", dict(lengths=[1500], hk=1, hv=3, g_low=-0.002, init_std=0.5)),
    ("prompt_4k", dict(lengths=[700], hk=2, hv=4, dk=64, dv=128, chunk=32, g_low=-0.01)),
]


def _out_tol(w, ro):
    """The outputs' max-abs bound.  With weak decay the outputs grow past the
    benchmark workloads' range and rounding them to bf16 alone moves them by
    up to |o| 2^-9; there the 2e-2 bound scales with max |o| / 2 (it is the
    plain bound wherever |o| <= 2)."""
    return U.BF16_OUT_MAXABS * max(1.0, float(np.abs(ro).max()) / 2)


@pytest.mark.parametrize("name,kw", CASES, ids=[f"{n}-{i}" for i, (n, _) in enumerate(CASES)])
def test_two_level_vs_oracle(name, kw):
    w = W.make_workload(name, **kw)
    ro, rf = oracle.reference_workload(w)
    tol = _out_tol(w, ro)
    out2, fin2, _ = U.run_gpu(w, scan_split=G.SCAN_TWO_LEVEL)
    U.check_bf16(out2, fin2, ro, rf, label=f"two-level {name} {kw}", out_tol=tol)
    out1, fin1, _ = U.run_gpu(w, scan_split=G.SCAN_ONE_PASS)
    U.check_bf16(out1, fin1, ro, rf, label=f"one pass {name} {kw}", out_tol=tol)
    # the two schedules differ by rounding only
    U.say(f"  two-level vs one pass: out max-abs {U.max_abs(out2, out1):.3e}, "
          f"final rel-L2 {U.rel_l2(fin2, fin1):.3e}")


def test_two_level_uniform_batch_4d():
    """Three sequences of 256 tokens as [B, T/B, H, D] tensors (no cu_seqlens)."""
    w = W.make_workload("prompt_4k", lengths=[256, 256, 256], hk=2, hv=2, init_std=0.2)
    ro, rf = oracle.reference_workload(w)
    d = W.to_device(w)
    B, L = 3, 256
    v4 = lambda x: x.view(B, L, *x.shape[1:])  # noqa: E731
    lay = G.gdn_get_workspace_layout(v4(d["q"]), v4(d["k"]), v4(d["v"]),
                                     opts=G.options(scan_split=G.SCAN_TWO_LEVEL))
    assert lay.split_chunks == 2  # (17 x 4 + 16) // 32
    U.say("  gpu run: uniform batch 3 x 256 as 4-D, two-level")
    G.gdn_prefill_ex(v4(d["q"]), v4(d["k"]), v4(d["v"]), v4(d["g"]), v4(d["beta"]), None,
                     d["init_state"], v4(d["out"]), d["final_state"],
                     opts=G.options(scan_split=G.SCAN_TWO_LEVEL))
    torch.cuda.synchronize()
    U.check_bf16(d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf,
                 label="uniform batch 4-D two-level")


def test_two_level_without_final_state():
    w = W.make_workload("prompt_4k", lengths=[640], hk=2, hv=2)
    ro, rf = oracle.reference_workload(w)
    d = W.to_device(w)
    U.say("  gpu run: two-level, no final state")
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None, d["out"], None,
                     opts=G.options(scan_split=G.SCAN_TWO_LEVEL))
    torch.cuda.synchronize()
    out = d["out"].float().cpu().numpy()
    ea = U.max_abs(out, ro)
    U.say(f"  out max-abs {ea:.3e}")
    assert np.isfinite(out).all() and ea <= U.BF16_OUT_MAXABS


def test_prompt_4k_full_two_level():
    """The 4096-token prompt split at chunk 34."""
    w = W.make_workload("prompt_4k")
    d = W.to_device(w)
    lay = G.gdn_get_workspace_layout(d["q"], d["k"], d["v"], opts=G.options(scan_split=G.SCAN_TWO_LEVEL))
    assert lay.split_chunks == 34  # (17 x 64 + 16) // 32
    ro, rf = oracle.reference_workload(w)
    out2, fin2, _ = U.run_gpu(w, dev=d, scan_split=G.SCAN_TWO_LEVEL)
    U.check_bf16(out2, fin2, ro, rf, label="prompt_4k full, two-level")
