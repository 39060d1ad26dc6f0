"""Every entry point on a stream other than the current one (GPU).

The library enqueues all of its work on the stream it is given; the binding
passes that stream through and, when it allocates a temporary workspace,
ties the block's lifetime to that stream.  Each call here runs on a side
stream (default priority) and must equal, bit for bit, the same call on the
current stream; the temporary workspace case also allocates and overwrites
memory on the current stream while the side stream's kernels run, which
would corrupt the result if the block were handed out again too early.
One graph cache is also shared by four threads with a stream each.
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


def _inputs():
    w = W.make_workload("long_16k_gqa", lengths=[900], hk=2, hv=4)
    return w, W.to_device(w)


def test_prefill_ex_on_a_side_stream():
    w, d = _inputs()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"])
    ref_o, ref_f = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(*args, ref_o, ref_f)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        o, f = torch.full_like(d["out"], 7.0), torch.full_like(d["final_state"], 7.0)
        torch.cuda.synchronize()
        # no workspace given: the binding allocates one for this call
        G.gdn_prefill_ex(*args, o, f, stream=side)
        # meanwhile the current stream allocates and overwrites memory
        junk = [torch.full((1 << 22,), float(rep), device="cuda") for _ in range(8)]
        del junk
        side.synchronize()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(f, ref_f), f"repetition {rep}"


def test_allocating_and_noalloc_entries_on_a_side_stream():
    w, d = _inputs()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"])
    ref_o, ref_f = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill(*args, ref_o, ref_f)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for entry in (G.gdn_prefill, G.gdn_prefill_noalloc):
        o, f = torch.full_like(d["out"], 7.0), torch.full_like(d["final_state"], 7.0)
        torch.cuda.synchronize()
        entry(*args, o, f, stream=side)
        side.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(f, ref_f), entry.__name__


def test_decode_and_output_gate_on_a_side_stream():
    w = W.make_workload("long_16k_gqa", lengths=[1] * 5, hk=2, hv=4, init_std=0.5)
    dev = {x: getattr(w, x).cuda() for x in ("q", "k", "v", "g", "beta")}
    s_ref, s_side = w.init_state.clone().cuda(), w.init_state.clone().cuda()
    o_ref = G.gdn_decode(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s_ref)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    o_side = torch.full_like(o_ref, 7.0)
    torch.cuda.synchronize()
    G.gdn_decode(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], s_side, out=o_side, stream=side)
    side.synchronize()
    assert torch.equal(o_side, o_ref) and torch.equal(s_side, s_ref)
    x, z, wn = (t.cuda() for t in W.make_gate_rows(64, 4, 128))
    y_ref = G.gdn_output_gate(x, z, wn)
    torch.cuda.synchronize()
    y_side = torch.full_like(y_ref, 7.0)
    torch.cuda.synchronize()
    G.gdn_output_gate(x, z, wn, out=y_side, stream=side)
    side.synchronize()
    assert torch.equal(y_side, y_ref)


def test_graph_replays_on_a_side_stream():
    w, d = _inputs()
    opts = G.options(chunk=64)
    ref_o, ref_f = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], ref_o, ref_f,
                     opts=opts)
    torch.cuda.synchronize()
    ws = G.alloc_workspace(d["q"], d["k"], d["v"], None, opts)
    cache = G.GraphCache(capacity=2)
    side = torch.cuda.Stream()
    for it in range(3):
        d["out"].fill_(7.0)
        d["final_state"].fill_(7.0)
        torch.cuda.synchronize()
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], d["out"],
                      d["final_state"], opts=opts, workspace=ws, stream=side)
        side.synchronize()
        assert torch.equal(d["out"], ref_o) and torch.equal(d["final_state"], ref_f), f"replay {it}"
    st = cache.stats()
    assert st["misses"] == 1 and st["hits"] == 2 and st["fallbacks"] == 0
    cache.close()


def test_one_graph_cache_shared_by_threads():
    """Four threads share one cache, each with its own buffers, workspace and
    stream (calls into the cache are serialised by the library); every
    result is bit-equal to the eager call."""
    import threading
    w, d = _inputs()
    opts = G.options(chunk=64)
    ref_o, ref_f = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], ref_o, ref_f,
                     opts=opts)
    torch.cuda.synchronize()
    cache = G.GraphCache(capacity=8)
    errors = []

    def worker(tid):
        try:
            side = torch.cuda.Stream()
            with torch.cuda.stream(side):
                o, f = torch.empty_like(ref_o), torch.empty_like(ref_f)
                ws = G.alloc_workspace(d["q"], d["k"], d["v"], None, opts)
            side.synchronize()
            for it in range(5):
                with torch.cuda.stream(side):
                    o.fill_(7.0)
                    f.fill_(7.0)
                cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], o, f,
                              opts=opts, workspace=ws, stream=side)
                side.synchronize()
                if not (torch.equal(o, ref_o) and torch.equal(f, ref_f)):
                    errors.append(f"thread {tid}, call {it}")
        except Exception as e:  # reported below
            errors.append(f"thread {tid}: {e!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    st = cache.stats()
    assert st["misses"] == 4 and st["hits"] == 16 and st["fallbacks"] == 0, st
    cache.close()
