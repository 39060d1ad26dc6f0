"""Captured replays (gdn_prefill_graph) against eager launches (GPU).

Each replay runs after eager work of the program itself (new inputs copied
into the captured buffers, an eager prefill into separate outputs, a
synchronisation), and every replay is compared with the eager result on
the same inputs: the same kernels on the same data, so bit for bit.
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


def _copy_inputs(dst, w):
    for name in ("q", "k", "v", "g", "beta"):
        dst[name].copy_(getattr(w, name).to(dst[name].device))
    if dst.get("init_state") is not None and w.init_state is not None:
        dst["init_state"].copy_(w.init_state.to(dst["init_state"].device))


def test_graph_replays_match_eager():
    kw = dict(lengths=[300], hk=2, hv=4, dk=128, dv=64)
    w0 = W.make_workload("long_16k_gqa", seed=0, **kw)
    d = W.to_device(w0)
    opts = G.options(chunk=64)
    ws = G.alloc_workspace(d["q"], d["k"], d["v"], None, opts)
    out_e, fin_e = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    cache = G.GraphCache(capacity=8)
    for it in range(4):
        w = W.make_workload("long_16k_gqa", seed=10 + it, **kw)
        _copy_inputs(d, w)
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"],
                         out_e, fin_e, opts=opts, workspace=ws)
        torch.cuda.synchronize()
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"],
                      d["out"], d["final_state"], opts=opts, workspace=ws)
        torch.cuda.synchronize()
        U.say(f"  replay {it}: {cache.stats()}")
        assert torch.equal(d["out"], out_e), f"replay {it}: output differs from eager"
        assert torch.equal(d["final_state"], fin_e), f"replay {it}: state differs from eager"
        if it == 3:
            ro, rf = oracle.reference_workload(w)
            U.check_bf16(d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf,
                         "replay vs oracle")
    st = cache.stats()
    assert st["misses"] == 1 and st["hits"] == 3 and st["entries"] == 1 and st["fallbacks"] == 0
    cache.close()


def test_graph_replay_follows_new_lengths():
    """The chunk table is rebuilt on the device at every replay, so a capture
    taken with one length mix serves another with the same T and N."""
    mixes = [[70, 1, 129], [100, 100, 0], [1, 198, 1], [200, 0, 0]]
    w0 = W.make_workload("edge_mix", lengths=mixes[0], hk=1, hv=2, dk=64, dv=64)
    d = W.to_device(w0)
    opts = G.options(chunk=64)
    ws = G.alloc_workspace(d["q"], d["k"], d["v"], d["cu_seqlens"], opts)
    out_e, fin_e = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    cache = G.GraphCache()
    for i, lens in enumerate(mixes):
        w = W.make_workload("edge_mix", seed=i, lengths=lens, hk=1, hv=2, dk=64, dv=64)
        _copy_inputs(d, w)
        d["cu_seqlens"].copy_(w.cu_seqlens.to(d["cu_seqlens"].device))
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], None,
                         out_e, fin_e, opts=opts, workspace=ws)
        torch.cuda.synchronize()
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], None,
                      d["out"], d["final_state"], opts=opts, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(d["out"], out_e) and torch.equal(d["final_state"], fin_e), lens
        ro, rf = oracle.reference_workload(w)
        U.check_bf16(d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf,
                     f"lengths {lens}")
    st = cache.stats()
    assert st["misses"] == 1 and st["hits"] == len(mixes) - 1
    cache.close()


def test_graph_cache_evicts_least_recently_used():
    w = W.make_workload("prompt_4k", lengths=[64], hk=1, hv=1, dk=32, dv=32)
    d = W.to_device(w)
    ws = G.alloc_workspace(d["q"], d["k"], d["v"])
    outs = [torch.empty_like(d["out"]) for _ in range(3)]
    cache = G.GraphCache(capacity=2)
    for o in outs + [outs[0]]:  # the fourth call's entry was evicted by the third
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], out=o, workspace=ws)
    cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], out=outs[0], workspace=ws)
    torch.cuda.synchronize()
    st = cache.stats()
    U.say(f"  {st}")
    assert st == {"entries": 2, "hits": 1, "misses": 4, "updates": 0, "fallbacks": 0}
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    cache.clear()
    assert cache.stats()["entries"] == 0
    cache.close()


def test_graph_cache_updates_for_fresh_buffers():
    """Twelve calls of one shape, each on fresh input and output buffers,
    enqueued with no synchronisation between them: the first four are
    instantiated, the other eight update the least recently used of them in
    place (their earlier launches may still be queued).  Every result is bit
    for bit the eager call's on the same buffers."""
    kw = dict(lengths=[256], hk=2, hv=2)
    sets = []
    for it in range(12):
        w = W.make_workload("prompt_4k", seed=40 + it, init_std=0.3, **kw)
        d = W.to_device(w)
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"],
                         d["out"], d["final_state"])
        sets.append((d, d["out"].clone(), d["final_state"].clone()))
    torch.cuda.synchronize()
    ws = G.alloc_workspace(sets[0][0]["q"], sets[0][0]["k"], sets[0][0]["v"])
    cache = G.GraphCache(capacity=8)
    for d, _, _ in sets:
        d["out"].fill_(7.0)
        d["final_state"].fill_(7.0)
    torch.cuda.synchronize()
    for d, _, _ in sets:
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], d["out"],
                      d["final_state"], workspace=ws)
    torch.cuda.synchronize()
    st = cache.stats()
    U.say(f"  {st}")
    for it, (d, eo, ef) in enumerate(sets):
        assert torch.equal(d["out"], eo) and torch.equal(d["final_state"], ef), f"call {it}"
    assert st == {"entries": 4, "hits": 0, "misses": 4, "updates": 8, "fallbacks": 0}
    cache.close()


def test_graph_cache_alternating_buffers_hit():
    """Two buffer sets used in turn (double buffering) stay two stored
    graphs: after the first call on each, every call is a hit."""
    kw = dict(lengths=[200], hk=2, hv=2)
    sets = []
    for it in range(2):
        w = W.make_workload("prompt_4k", seed=60 + it, **kw)
        d = W.to_device(w)
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None, d["out"], d["final_state"])
        sets.append((d, d["out"].clone(), d["final_state"].clone()))
    torch.cuda.synchronize()
    ws = G.alloc_workspace(sets[0][0]["q"], sets[0][0]["k"], sets[0][0]["v"])
    cache = G.GraphCache(capacity=8)
    for it in range(6):
        d, eo, ef = sets[it % 2]
        d["out"].fill_(7.0)
        d["final_state"].fill_(7.0)
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None, d["out"],
                      d["final_state"], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(d["out"], eo) and torch.equal(d["final_state"], ef), f"call {it}"
    assert cache.stats() == {"entries": 2, "hits": 4, "misses": 2, "updates": 0, "fallbacks": 0}
    cache.close()


def test_graph_replays_two_level_scan_and_beta_logits():
    """The two-level scan (two scan launches, its workspace regions) and the
    write gate given as logits, captured once and replayed on new inputs:
    bit for bit the eager result each time, and the oracle on the last."""
    kw = dict(lengths=[640], hk=2, hv=4, g_low=-0.02)
    w0 = W.make_workload("prompt_4k", seed=0, **kw)
    d = W.to_device(w0)
    opts = G.options(chunk=64, scan_split=G.SCAN_TWO_LEVEL, beta_logits=True)
    ws = G.alloc_workspace(d["q"], d["k"], d["v"], None, opts)
    assert G.gdn_get_workspace_layout(d["q"], d["k"], d["v"], opts=opts).split_chunks > 0
    out_e, fin_e = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    cache = G.GraphCache(capacity=4)
    for it in range(3):
        w = W.make_workload("prompt_4k", seed=20 + it, **kw)
        _copy_inputs(d, w)
        b = w.beta.double().numpy()
        d["beta"].copy_(torch.from_numpy((np.log(b) - np.log1p(-b)).astype(np.float32)))
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"],
                         out_e, fin_e, opts=opts, workspace=ws)
        torch.cuda.synchronize()
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"],
                      d["out"], d["final_state"], opts=opts, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(d["out"], out_e) and torch.equal(d["final_state"], fin_e), it
    ro, rf = oracle.reference_workload(w)
    U.check_bf16(d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf,
                 "two-level replay vs oracle", out_tol=U.BF16_OUT_MAXABS * max(1.0, float(np.abs(ro).max()) / 2))
    st = cache.stats()
    assert st["misses"] == 1 and st["hits"] == 2 and st["fallbacks"] == 0
    cache.close()
