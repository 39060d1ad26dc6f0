"""Element offsets past 2^31 (GPU).

A batch of 1100 sequences of 1024 tokens, 16 heads, d = 128 (bf16): every
[T, H, d] tensor holds 2.3e9 elements, so the last sequence's rows start
past element 2^31 of q, k, v and out, and its intermediates past 2^31
elements of the workspace.  Only the last sequence holds seeded data (a
reduced prompt workload); the others are zero rows, whose outputs and final
states are exactly zero.  The last sequence is compared with the float64
oracle at the bf16 tolerances, once as a uniform [B, T, H, d] batch and
once packed with cu_seqlens.  About 40 GB of device memory.
"""
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

B, L, H, D = 1100, 1024, 16, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()
    oracle.load()


def test_offsets_past_2_pow_31():
    assert (B - 1) * L * H * D > 2 ** 31
    w = W.make_workload("prompt_4k", lengths=[L])
    ro, rf = oracle.reference_workload(w)
    dev = torch.device("cuda")
    q = torch.zeros(B, L, H, D, dtype=torch.bfloat16, device=dev)
    k = torch.zeros_like(q)
    v = torch.zeros_like(q)
    g = torch.zeros(B, L, H, dtype=torch.float32, device=dev)
    beta = torch.zeros_like(g)
    q[B - 1].copy_(w.q.to(dev))
    k[B - 1].copy_(w.k.to(dev))
    v[B - 1].copy_(w.v.to(dev))
    g[B - 1].copy_(w.g.to(dev))
    beta[B - 1].copy_(w.beta.to(dev))
    fin = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device=dev)
    for packed in (False, True):
        out = torch.full_like(q, 7.0)
        fin.fill_(7.0)
        U.say(f"  {B} x {L} tokens x {H} heads, packed={packed}")
        if packed:
            flat = lambda t: t.reshape(B * L, *t.shape[2:])  # noqa: E731
            G.gdn_prefill_ex(flat(q), flat(k), flat(v), flat(g), flat(beta), cu, None, flat(out), fin)
        else:
            G.gdn_prefill_ex(q, k, v, g, beta, None, None, out, fin)
        torch.cuda.synchronize()
        U.check_bf16(out[B - 1].float().cpu().numpy(), fin[B - 1:].cpu().numpy(), ro, rf,
                     label=f"last sequence, packed={packed}")
        # zero rows give zero outputs and states, here and just before the last
        for s in (0, B // 2, B - 2):
            assert torch.count_nonzero(out[s]) == 0 and torch.count_nonzero(fin[s]) == 0, s
        del out
        torch.cuda.empty_cache()


def test_decode_state_past_2_pow_31():
    """Decode over 8500 sequences x 16 heads: the f32 state holds 2.2e9
    elements (8.9 GB), the last sequence's past element 2^31; only it holds
    seeded data."""
    N = 8500
    assert (N - 1) * H * D * D > 2 ** 31
    w = W.make_workload("prompt_4k", lengths=[1], init_std=0.5)
    ro, rf = oracle.reference_workload(w)
    dev = torch.device("cuda")
    q = torch.zeros(N, H, D, dtype=torch.bfloat16, device=dev)
    k, v = torch.zeros_like(q), torch.zeros_like(q)
    g = torch.zeros(N, H, dtype=torch.float32, device=dev)
    beta = torch.zeros_like(g)
    state = torch.zeros(N, H, D, D, dtype=torch.float32, device=dev)
    for dst, src in ((q, w.q), (k, w.k), (v, w.v), (g, w.g), (beta, w.beta)):
        dst[N - 1].copy_(src[0].to(dev))
    state[N - 1].copy_(w.init_state[0].to(dev))
    out = G.gdn_decode(q, k, v, g, beta, state)
    torch.cuda.synchronize()
    es = U.rel_l2(state[N - 1:].cpu().numpy(), rf)
    eo = U.max_abs(out[N - 1:].float().cpu().numpy(), ro)
    U.say(f"  decode {N} x {H} heads: last sequence state rel-L2 {es:.3e}, out max-abs {eo:.3e}")
    assert es <= U.F32_RELL2 and eo <= 8e-3 * max(1.0, float(abs(ro).max()))
    for s in (0, N // 2, N - 2):
        assert torch.count_nonzero(out[s]) == 0 and torch.count_nonzero(state[s]) == 0, s
