"""A seeded sweep of the configuration space against the float64 oracle (GPU).

Each case draws, from its own seed: the input dtype, d_k and d_v (16 ..
128), key heads and the value heads per key head (1 .. 4), the chunk size,
1 .. 4 sequences of 1 .. 300 tokens (some at chunk multiples and one off
them) packed with cu_seqlens or passed as one sequence, the decay range,
the write gate's class mix, an initial state or none, the output scale,
and the steps fused into the loads (beta from logits, the decay from its
projection, silu, the short convolution with or without history).  The
reference applies the same steps with the float64 oracle functions to the
raw inputs and runs the oracle's recurrence; the prefill must meet the
tolerances of its dtype (bf16: max-abs 2e-2 on outputs, scaled with max |o|
/ 2 where weak decay lets |o| grow past 2, and rel-L2 5e-3 on the final
state; fp32: rel-L2 1e-5 on both).  Configurations the library does not
build (some fp32 chunk and d_k pairs) are drawn again.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import gates, oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

N_CASES = 300


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()
    oracle.load()


def draw(case: int):
    rng = np.random.default_rng([case, 0x5EE9])
    fp32 = rng.random() < 0.3
    chunk = int(rng.choice([16, 32] if fp32 else [16, 32, 64]))
    n = int(rng.integers(1, 5))
    lengths = []
    for _ in range(n):
        kind = rng.integers(0, 3)
        if kind == 0:
            lengths.append(int(rng.integers(1, 301)))
        elif kind == 1:
            lengths.append(int(chunk * rng.integers(1, 5)))
        else:
            lengths.append(int(chunk * rng.integers(1, 5) + rng.choice([-1, 1])))
    hk = int(rng.integers(1, 4))
    cfg = dict(
        spec=dict(lengths=lengths, hk=hk, hv=hk * int(rng.integers(1, 5)),
                  dk=int(rng.choice([16, 32, 64, 128])), dv=int(rng.choice([16, 32, 64, 128])),
                  chunk=chunk, dtype="fp32" if fp32 else "bf16",
                  g_low=float(rng.choice([-0.1, -1.0, -5.0])),
                  beta=str(rng.choice(["sigmoid_normal", "three_class"])),
                  init_std=0.3 if rng.random() < 0.5 else None),
        packed=n > 1 or rng.random() < 0.5,
        scale=float(rng.choice([1.0, 0.5, 2.0])),
        beta_logits=rng.random() < 0.25,
        decay_proj=rng.random() < 0.25,
        silu=rng.random() < 0.3,
        conv=int(rng.integers(1, 5)) if rng.random() < 0.3 else 0,
        conv_hist=rng.random() < 0.5,
    )
    return cfg


def available(cfg) -> bool:
    s = cfg["spec"]
    dt = torch.float32 if s["dtype"] == "fp32" else torch.bfloat16
    q = torch.empty(8, s["hk"], s["dk"], dtype=dt)
    v = torch.empty(8, s["hv"], s["dv"], dtype=dt)
    try:
        G.gdn_workspace_size(q, q, v, opts=G.options(chunk=s["chunk"]))
    except G.GdnError as e:
        if e.status == -5:  # GDN_ERR_UNSUPPORTED
            return False
        raise
    return True


def case_config(case: int):
    """The case's configuration: the first draw the library builds."""
    for attempt in range(50):
        cfg = draw(case + 1000 * attempt)
        if available(cfg):
            return cfg
    raise AssertionError("no buildable configuration drawn")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep(case):
    cfg = case_config(case)
    spec = cfg["spec"]
    w = W.make_workload("prompt_4k", seed=case, **spec)
    d = W.to_device(w)
    U.say(f"  sweep {case}: {spec} packed={cfg['packed']} scale={cfg['scale']} "
          f"logits={cfg['beta_logits']} proj={cfg['decay_proj']} silu={cfg['silu']} "
          f"conv={cfg['conv']} hist={cfg['conv_hist']}")
    extra, g_dev, b_dev = {}, d["g"], d["beta"]
    g_ref, b_ref = w.g, w.beta
    if cfg["decay_proj"]:
        gi = W.make_gate_inputs(w, seed=case)
        extra.update(decay_proj=True, decay_a_log=gi.a_log.cuda(), decay_bias=gi.bias.cuda())
        g_dev = gi.a.cuda()
        g_ref = torch.from_numpy(gates.decay_from_projection(gi.a, gi.a_log, gi.bias))
    if cfg["beta_logits"]:
        logit = torch.log(w.beta.double() / (1 - w.beta.double()))
        extra.update(beta_logits=True)
        b_dev = logit.float().cuda()
        b_ref = torch.from_numpy(gates.sigmoid(logit.float().double().numpy()))
    q, k, v = w.q, w.k, w.v
    if cfg["conv"]:
        taps, hist = W.make_conv_inputs(w, cfg["conv"], seed=case)
        hist_used = hist if cfg["conv_hist"] else None
        extra.update(conv_weight=taps.cuda(), conv_state_in=None if hist_used is None else hist.cuda())
        T = w.q.shape[0]
        X = torch.cat([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], 1).double().numpy()
        y, _ = gates.short_conv(X, taps.double().numpy(), w.lengths,
                                None if hist_used is None else hist_used.double().numpy())
        if cfg["silu"]:
            y = gates.silu(y)
        Y = torch.from_numpy(np.asarray(y, np.float64)).to(w.q.dtype)
        qk = w.q.shape[1] * w.q.shape[2]
        q, k, v = Y[:, :qk].reshape(q.shape), Y[:, qk:2 * qk].reshape(k.shape), Y[:, 2 * qk:].reshape(v.shape)
    elif cfg["silu"]:
        act = lambda x: torch.from_numpy(np.asarray(gates.silu(x.double().numpy()), np.float64)).to(x.dtype)  # noqa: E731
        q, k, v = act(q), act(k), act(v)
    if cfg["silu"]:
        extra.update(qkv_silu=True)
    opts = G.options(chunk=spec["chunk"], scale=cfg["scale"], **extra)
    cu = d["cu_seqlens"] if cfg["packed"] else None
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], g_dev, b_dev, cu, d["init_state"], d["out"],
                     d["final_state"], opts=opts)
    torch.cuda.synchronize()
    ro, rf = oracle.reference(q, k, v, g_ref, b_ref, w.lengths, w.init_state, scale=cfg["scale"])
    out, fin = d["out"].float().cpu().numpy(), d["final_state"].cpu().numpy()
    if w.q.dtype == torch.bfloat16:
        U.check_bf16(out, fin, ro, rf, label=f"sweep {case}",
                     out_tol=U.BF16_OUT_MAXABS * max(1.0, float(np.abs(ro).max()) / 2))
    else:
        U.check_f32(out, fin, ro, rf, label=f"sweep {case}")
