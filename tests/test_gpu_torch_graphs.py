"""The library's calls inside a caller's own captured graph (GPU).

A serving loop may capture its decode steps, or a prefill with a
preallocated workspace, in a torch CUDA graph (a HIP graph on ROCm).
Neither call allocates or clears memory with a memset in that form, so
both capture; each graph is replayed several times, with eager work of the
program and synchronisations between the replays, and every replay is
compared with the same calls run eagerly.
"""
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()


def test_decode_steps_in_a_captured_graph():
    """Four decode steps of 6 sequences (grouped heads, the short
    convolution and silu, the history updated in place) in one graph."""
    steps, N = 4, 6
    w = W.make_workload("long_16k_gqa", lengths=[steps] * N, hk=2, hv=4, init_std=0.5)
    taps, hist0 = W.make_conv_inputs(w, 4)
    # token t of every sequence: rows t, steps + t, ...
    tok = lambda x, t: x.reshape(N, steps, *x.shape[1:])[:, t].contiguous().cuda()  # noqa: E731
    xs = [{n: tok(getattr(w, n), t) for n in ("q", "k", "v", "g", "beta")} for t in range(steps)]
    tw = taps.cuda()

    def run(state, hist, outs):
        opts = G.options(qkv_silu=True, conv_weight=tw, conv_state_in=hist, conv_state_out=hist)
        for t in range(steps):
            x = xs[t]
            G.gdn_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], state, out=outs[t], opts=opts)

    e_state, e_hist = w.init_state.clone().cuda(), hist0.clone().cuda()
    e_outs = [torch.empty_like(xs[0]["v"]) for _ in range(steps)]
    run(e_state, e_hist, e_outs)
    torch.cuda.synchronize()

    g_state, g_hist = torch.empty_like(e_state), torch.empty_like(e_hist)
    g_outs = [torch.empty_like(o) for o in e_outs]
    g_state.copy_(w.init_state.cuda())
    g_hist.copy_(hist0.cuda())
    run(g_state, g_hist, g_outs)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            run(g_state, g_hist, g_outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        g_state.copy_(w.init_state.cuda())
        g_hist.copy_(hist0.cuda())
        for o in g_outs:
            o.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g_state, e_state) and torch.equal(g_hist, e_hist), f"replay {rep}"
        for t in range(steps):
            assert torch.equal(g_outs[t], e_outs[t]), f"replay {rep}, step {t}"
        # eager work of the program between replays
        run(torch.empty_like(e_state).copy_(e_state), torch.empty_like(e_hist).copy_(e_hist),
            [torch.empty_like(o) for o in e_outs])


@pytest.mark.parametrize("packed", [False, True])
def test_prefill_with_workspace_in_a_captured_graph(packed):
    w = W.make_workload("packed_255", lengths=[300, 17, 129], hk=2, hv=4) if packed else \
        W.make_workload("long_16k_gqa", lengths=[500], hk=2, hv=4)
    d = W.to_device(w)
    cu = d["cu_seqlens"] if packed else None
    opts = G.options(chunk=64)
    ws = G.alloc_workspace(d["q"], d["k"], d["v"], cu, opts)
    eo, ef = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"], eo, ef,
                     opts=opts, workspace=ws)
    torch.cuda.synchronize()
    o, f = torch.empty_like(eo), torch.empty_like(ef)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph):
            G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"], o, f,
                             opts=opts, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        o.fill_(7.0)
        f.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eo) and torch.equal(f, ef), f"replay {rep}"
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"],
                         torch.empty_like(eo), torch.empty_like(ef), opts=opts, workspace=ws)
