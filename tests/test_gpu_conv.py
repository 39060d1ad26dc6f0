"""GDN_FLAG_QKV_CONV (GPU): every channel of q, k and v passes through a
short causal depthwise convolution along its sequence's tokens, then silu
(with GDN_FLAG_QKV_SILU), rounded once to the input dtype, as the kernels
load the rows.

The reference is the float64 oracle run on oracle.gates.short_conv of the
raw rows (then oracle.gates.silu), rounded to the input dtype.  The kernel
forms the same sum in fp32; where the fp32 and float64 values fall on
opposite sides of a rounding boundary of the input dtype the two inputs
differ by one ulp, which the prefill's tolerances absorb.  Each case first
checks that the oracle on the raw inputs (no convolution) lands far outside
those tolerances, so a kernel that skipped the convolution, or applied it
to only some of q, k, v, could not pass.  The new history (conv_state_out)
holds raw rows, so it must equal the oracle's bit for bit.
"""
import dataclasses

import numpy as np
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import gates, oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()
    oracle.load()


def channels(w) -> torch.Tensor:
    """[T, D] rows of the channels q | k | v."""
    T = w.q.shape[0]
    return torch.cat([w.q.reshape(T, -1), w.k.reshape(T, -1), w.v.reshape(T, -1)], 1)


def conv_inputs(w, taps, hist, silu, lengths=None):
    """q, k, v after the convolution (and silu), rounded to their dtype, and
    the new history (float64), from the float64 oracle functions."""
    st = None if hist is None else hist.double().numpy()
    y, fin = gates.short_conv(channels(w).double().numpy(), taps.double().numpy(),
                              w.lengths if lengths is None else lengths, st)
    if silu:
        y = gates.silu(y)
    Y = torch.from_numpy(np.asarray(y, np.float64)).to(w.q.dtype)
    qk = w.q.shape[1] * w.q.shape[2]
    return (Y[:, :qk].reshape(w.q.shape), Y[:, qk:2 * qk].reshape(w.k.shape),
            Y[:, 2 * qk:].reshape(w.v.shape), fin)


def conv_reference(w, taps, hist, silu):
    q, k, v, fin = conv_inputs(w, taps, hist, silu)
    ro, rf = oracle.reference(q, k, v, w.g, w.beta, w.lengths, w.init_state)
    return ro, rf, fin


def check(w, out, fin, ro, rf, label):
    # the test's power: the plain recurrence on the raw inputs is far off
    po, pf = oracle.reference_workload(w)
    if w.q.dtype == torch.bfloat16:
        assert U.max_abs(po, ro) > 10 * U.BF16_OUT_MAXABS or U.rel_l2(pf, rf) > 10 * U.BF16_STATE_RELL2
        U.check_bf16(out, fin, ro, rf, label=label)
    else:
        assert U.rel_l2(po, ro) > 1e3 * U.F32_RELL2
        U.check_f32(out, fin, ro, rf, label=label)


def history_equal(got: torch.Tensor, want: np.ndarray, label: str):
    want_t = torch.from_numpy(np.asarray(want, np.float64)).to(got.dtype)
    assert torch.equal(got.cpu(), want_t), f"{label}: new history differs"


CASES = [
    # (workload, overrides, width, silu, history given, extra options)
    ("prompt_4k", dict(lengths=[700], hk=2, hv=4), 4, True, True, {}),
    ("long_16k_gqa", dict(lengths=[300], hk=2, hv=6), 4, True, True, {}),        # grouped heads
    ("packed_255", dict(lengths=("uniform", 12, 1, 200), hk=2, hv=2), 4, True, True, {}),
    ("edge_mix", dict(hk=1, hv=2), 3, True, False, {}),                          # ragged, fresh
    ("prompt_4k", dict(lengths=[333], hk=2, hv=2, dk=64, dv=64, chunk=32), 2, True, True, {}),
    ("prompt_4k", dict(lengths=[200], hk=1, hv=2, dk=32, dv=128, chunk=16), 4, True, True, {}),
    ("tiny_fp32", dict(lengths=[150], hk=2, hv=4, dk=64, dv=32, chunk=32), 4, True, True, {}),
    ("tiny_fp32", dict(lengths=[90, 1, 41], hk=1, hv=3, dk=32, dv=64, chunk=16), 3, True, True, {}),
    ("edge_mix", dict(lengths=[0, 2, 1, 0, 130], hk=2, hv=2), 4, True, True, {}),  # empty, 1, 2 tokens
    ("prompt_4k", dict(lengths=[500], hk=2, hv=4), 4, False, True, {}),          # no silu
    ("prompt_4k", dict(lengths=[300], hk=2, hv=2), 1, True, False, {}),          # width 1
    ("prompt_4k", dict(lengths=[1000], hk=2, hv=4), 4, True, True, dict(segment_chunks=3)),
    ("prompt_4k", dict(lengths=[900], hk=2, hv=2), 4, True, True, dict(scan_split=G.SCAN_TWO_LEVEL)),
]


@pytest.mark.parametrize("name,kw,width,silu,with_hist,extra", CASES,
                         ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_prefill_with_conv(name, kw, width, silu, with_hist, extra):
    w = W.make_workload(name, **kw)
    taps, hist = W.make_conv_inputs(w, width)
    d = W.to_device(w)
    cu = d["cu_seqlens"] if w.n_seqs > 1 else None
    h_in = hist.cuda() if with_hist else None
    h_out = torch.full_like(hist, 7.0).cuda()
    opts = G.options(chunk=w.chunk, qkv_silu=silu, conv_weight=taps.cuda(), conv_state_in=h_in,
                     conv_state_out=h_out, **extra)
    U.say(f"  conv {name} {kw} width {width} silu {silu} history {with_hist} {extra}")
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"],
                     d["out"], d["final_state"], opts=opts)
    torch.cuda.synchronize()
    ro, rf, rh = conv_reference(w, taps, hist if with_hist else None, silu)
    check(w, d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf,
          f"conv {name} {kw} w{width}")
    if width > 1:
        history_equal(h_out, rh, name)


def test_prompt_4k_full_with_conv():
    """The throughput workload at full size (4096 tokens, 16 heads, d = 128)
    with the convolution and silu, compared in full."""
    w = W.make_workload("prompt_4k")
    taps, hist = W.make_conv_inputs(w, 4)
    d = W.to_device(w)
    h_out = torch.empty_like(hist).cuda()
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, None, d["out"], d["final_state"],
                     opts=G.options(qkv_silu=True, conv_weight=taps.cuda(), conv_state_in=hist.cuda(),
                                    conv_state_out=h_out))
    torch.cuda.synchronize()
    ro, rf, rh = conv_reference(w, taps, hist, True)
    check(w, d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy(), ro, rf, "conv prompt_4k full")
    history_equal(h_out, rh, "prompt_4k full")


def test_uniform_batch_and_in_place_history():
    """[B, T, H, d] inputs without cu_seqlens (sequences at the batch
    stride), the history read and rewritten in place."""
    B, L = 3, 260
    w = W.make_workload("prompt_4k", lengths=[L] * B, hk=2, hv=2)
    taps, hist = W.make_conv_inputs(w, 4)
    d = W.to_device(w)
    q4, k4, v4 = (d[n].reshape(B, L, *d[n].shape[1:]) for n in ("q", "k", "v"))
    g4, b4 = d["g"].reshape(B, L, -1), d["beta"].reshape(B, L, -1)
    o4 = torch.empty_like(v4)
    f4 = torch.empty_like(d["final_state"])
    h = hist.clone().cuda()
    G.gdn_prefill_ex(q4, k4, v4, g4, b4, None, None, o4, f4,
                     opts=G.options(qkv_silu=True, conv_weight=taps.cuda(), conv_state_in=h,
                                    conv_state_out=h))
    torch.cuda.synchronize()
    w0 = dataclasses.replace(w, init_state=None)
    ro, rf, rh = conv_reference(w0, taps, hist, True)
    check(w0, o4.reshape(d["out"].shape).float().cpu().numpy(), f4.cpu().numpy(), ro, rf,
          "conv uniform batch")
    history_equal(h, rh, "in place")


def test_prefill_in_two_calls():
    """A prompt in two calls, the state and the history carried, against
    the oracle over the whole prompt."""
    w = W.make_workload("long_16k_gqa", lengths=[700], hk=2, hv=4)
    taps, hist = W.make_conv_inputs(w, 4)
    ro, rf, rh = conv_reference(w, taps, hist, True)
    d = W.to_device(w)
    tw = taps.cuda()
    for cut in (128, 301):
        h = hist.clone().cuda()
        st = d["init_state"].clone()
        out = torch.empty_like(d["out"])
        for lo, hi in ((0, cut), (cut, 700)):
            G.gdn_prefill_ex(d["q"][lo:hi], d["k"][lo:hi], d["v"][lo:hi], d["g"][lo:hi],
                             d["beta"][lo:hi], None, st, out[lo:hi], st,
                             opts=G.options(qkv_silu=True, conv_weight=tw, conv_state_in=h,
                                            conv_state_out=h))
        torch.cuda.synchronize()
        U.check_bf16(out.float().cpu().numpy(), st.cpu().numpy(), ro, rf, label=f"two calls, cut {cut}")
        history_equal(h, rh, f"two calls, cut {cut}")


def test_segments_bit_identical_with_conv():
    """Segments read the history of a later segment's first chunk from the
    input rows before it: bit for bit the one-pass call."""
    w = W.make_workload("prompt_4k", lengths=[1100], hk=2, hv=4)
    taps, hist = W.make_conv_inputs(w, 4)
    d = W.to_device(w)
    res = []
    for seg in (-1, 2, 5):
        o = torch.full_like(d["out"], 7.0)
        f = torch.full_like(d["final_state"], 7.0)
        h = torch.full_like(hist, 7.0).cuda()
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], o, f,
                         opts=G.options(qkv_silu=True, conv_weight=taps.cuda(),
                                        conv_state_in=hist.cuda(), conv_state_out=h,
                                        segment_chunks=seg))
        torch.cuda.synchronize()
        res.append((o, f, h))
    for o, f, h in res[1:]:
        assert torch.equal(o, res[0][0]) and torch.equal(f, res[0][1]) and torch.equal(h, res[0][2])


def test_conv_with_every_gate():
    """The convolution with the decay projection, beta logits and the gated
    output norm in one call: the final state against the oracle, the outputs
    bit-equal to the same call without the output gate followed by
    gdn_output_gate."""
    w = W.make_workload("prompt_4k", lengths=[400], hk=2, hv=4)
    taps, hist = W.make_conv_inputs(w, 4)
    d = W.to_device(w)
    gi = W.make_gate_inputs(w)
    g_ref = gates.decay_from_projection(gi.a, gi.a_log, gi.bias)
    b_logit = torch.log(w.beta / (1 - w.beta))
    z = gi.z.cuda()
    base = dict(qkv_silu=True, conv_weight=taps.cuda(), conv_state_in=hist.cuda(), decay_proj=True,
                decay_a_log=gi.a_log.cuda(), decay_bias=gi.bias.cuda(), beta_logits=True)
    o1, f1 = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], gi.a.cuda(), b_logit.float().cuda(), None, None, o1, f1,
                     opts=G.options(**base, gate_z=z, norm_weight=gi.norm_w.cuda()))
    o2, f2 = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], gi.a.cuda(), b_logit.float().cuda(), None, None, o2, f2,
                     opts=G.options(**base))
    G.gdn_output_gate(o2, z, gi.norm_w.cuda(), out=o2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(f1, f2)
    q, k, v, _ = conv_inputs(w, taps, hist, True)
    _, rf = oracle.reference(q, k, v, g_ref, gates.sigmoid(b_logit.double().numpy()), w.lengths, None)
    es = U.rel_l2(f1.cpu().numpy(), rf)
    U.say(f"  conv + every gate: final rel-L2 {es:.3e}")
    assert es <= U.BF16_STATE_RELL2


DECODE_CASES = [
    ("bf16-gqa", "long_16k_gqa", 9, dict(hk=2, hv=6, dk=128, dv=64), True),
    ("bf16-d128", "prompt_4k", 4, dict(hk=4, hv=4, dk=128, dv=128), True),
    ("bf16-noact", "prompt_4k", 3, dict(hk=2, hv=2, dk=64, dv=32), False),
    ("f32-d64", "tiny_fp32", 5, dict(hk=2, hv=4, dk=64, dv=32), True),
]


@pytest.mark.parametrize("label,name,n,kw,silu", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_with_conv(label, name, n, kw, silu):
    """One token per sequence; the history read and shifted in place.  The
    state's bound for bf16 inputs is the prefill's (5e-3 rel-L2): the
    convolved inputs are rounded values, where a rounding boundary can flip
    one ulp, unlike the decode tests on raw inputs."""
    w = W.make_workload(name, lengths=[1] * n, init_std=0.5, **kw)
    taps, hist = W.make_conv_inputs(w, 4)
    dev = {x: getattr(w, x).cuda() for x in ("q", "k", "v", "g", "beta")}
    state = w.init_state.clone().cuda()
    h = hist.clone().cuda()
    out = G.gdn_decode(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], state,
                       opts=G.options(qkv_silu=silu, conv_weight=taps.cuda(), conv_state_in=h,
                                      conv_state_out=h))
    torch.cuda.synchronize()
    ro, rf, rh = conv_reference(w, taps, hist, silu)
    po, _ = oracle.reference_workload(w)
    got_o, got_s = out.float().cpu().numpy(), state.cpu().numpy()
    es = U.rel_l2(got_s, rf)
    U.say(f"  decode conv {label}: state rel-L2 {es:.3e}")
    history_equal(h, rh, label)
    if w.q.dtype == torch.bfloat16:
        assert U.max_abs(po, ro) > 0.1 * max(1.0, float(np.abs(ro).max()))
        assert es <= U.BF16_STATE_RELL2
        assert U.max_abs(got_o, ro) <= 8e-3 * max(1.0, float(np.abs(ro).max()))
    else:
        assert U.rel_l2(po, ro) > 1e-2
        assert es <= U.F32_RELL2 and U.rel_l2(got_o, ro) <= U.F32_RELL2


def test_decode_continues_the_prefill():
    """A prefill of L tokens (state and history out), then decode steps,
    against one prefill of all the tokens."""
    L, n = 200, 6
    w = W.make_workload("prompt_4k", lengths=[L + n], hk=2, hv=4, init_std=0.1)
    taps, hist = W.make_conv_inputs(w, 4)
    d = W.to_device(w)
    tw = taps.cuda()
    full_o = torch.empty_like(d["out"])
    full_f = torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], full_o, full_f,
                     opts=G.options(qkv_silu=True, conv_weight=tw, conv_state_in=hist.cuda()))
    h = hist.clone().cuda()
    st = d["init_state"].clone()
    o = torch.empty_like(d["out"])
    G.gdn_prefill_ex(d["q"][:L], d["k"][:L], d["v"][:L], d["g"][:L], d["beta"][:L], None, st, o[:L], st,
                     opts=G.options(qkv_silu=True, conv_weight=tw, conv_state_in=h, conv_state_out=h))
    for t in range(L, L + n):
        G.gdn_decode(d["q"][t:t + 1], d["k"][t:t + 1], d["v"][t:t + 1], d["g"][t:t + 1],
                     d["beta"][t:t + 1], st, out=o[t:t + 1],
                     opts=G.options(qkv_silu=True, conv_weight=tw, conv_state_in=h, conv_state_out=h))
    torch.cuda.synchronize()
    ea = U.max_abs(o.float().cpu().numpy(), full_o.float().cpu().numpy())
    es = U.rel_l2(st.cpu().numpy(), full_f.cpu().numpy())
    U.say(f"  prefill + decode against one prefill: out max-abs {ea:.3e}, state rel-L2 {es:.3e}")
    assert ea <= U.BF16_OUT_MAXABS and es <= U.BF16_STATE_RELL2
    _, _, rh = conv_reference(w, taps, hist, True)
    history_equal(h, rh, "after the decode steps")


def test_conv_in_graph_replays():
    """Captured calls with the convolution replay bit for bit the eager call
    (the history output rewritten on every replay)."""
    w = W.make_workload("long_16k_gqa", lengths=[300], hk=2, hv=4)
    taps, hist = W.make_conv_inputs(w, 4)
    d = W.to_device(w)
    h_in, h_out = hist.cuda(), torch.empty_like(hist).cuda()
    opts = G.options(chunk=64, qkv_silu=True, conv_weight=taps.cuda(), conv_state_in=h_in,
                     conv_state_out=h_out)
    eo, ef = torch.empty_like(d["out"]), torch.empty_like(d["final_state"])
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"], eo, ef, opts=opts)
    torch.cuda.synchronize()
    eh = h_out.clone()
    ws = G.alloc_workspace(d["q"], d["k"], d["v"], None, opts)
    cache = G.GraphCache(capacity=2)
    for it in range(3):
        d["out"].fill_(7.0)
        d["final_state"].fill_(7.0)
        h_out.fill_(7.0)
        cache.prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, d["init_state"],
                      d["out"], d["final_state"], opts=opts, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(d["out"], eo) and torch.equal(d["final_state"], ef), f"replay {it}"
        assert torch.equal(h_out, eh), f"replay {it}: history"
    st = cache.stats()
    assert st["misses"] == 1 and st["hits"] == 2 and st["fallbacks"] == 0
    cache.close()
