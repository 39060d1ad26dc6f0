"""Helpers shared by the GPU tests (not collected by pytest)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W

# Tolerances stated for the prefill: bf16 inputs -> max-abs error of the
# outputs <= 2e-2 and relative L2 error of the fp32 final state <= 5e-3;
# fp32 inputs -> relative L2 error <= 1e-5 (outputs and final state).
BF16_OUT_MAXABS = 2e-2
BF16_STATE_RELL2 = 5e-3
F32_RELL2 = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def max_abs(a, b) -> float:
    return float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).max()) if np.size(a) else 0.0


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a - b))


def run_gpu(w: W.Workload, chunk=None, scale=1.0, with_cu=None, entry="ex",
            init_alias=False, dev=None, scan_split=0):
    """Run the library on a workload; returns (out f32 numpy, final numpy,
    device tensors)."""
    d = dev if dev is not None else W.to_device(w)
    if with_cu is None:
        with_cu = w.n_seqs > 1
    cu = d["cu_seqlens"] if with_cu else None
    fin = d["final_state"]
    if init_alias:
        assert d["init_state"] is not None
        fin = d["init_state"]
    say(f"  gpu run: {w.name} T={w.t_total} N={w.n_seqs} Hk={w.q.shape[1]} "
        f"Hv={w.v.shape[1]} dk={w.q.shape[2]} dv={w.v.shape[2]} "
        f"dtype={w.q.dtype} chunk={chunk or w.chunk} entry={entry} scan_split={scan_split}")
    if entry == "ex":
        G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu,
                         d["init_state"], d["out"], fin,
                         opts=G.options(chunk=chunk or w.chunk, scale=scale, scan_split=scan_split))
    else:
        assert (chunk or w.chunk) == 64 or w.q.dtype != torch.bfloat16
        G.gdn_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], cu,
                      d["init_state"], d["out"], fin)
    torch.cuda.synchronize()
    return (d["out"].float().cpu().numpy(), fin.cpu().numpy(), d)


def check_bf16(out, fin, ref_out, ref_fin, label="", out_tol=BF16_OUT_MAXABS):
    ea = max_abs(out, ref_out)
    es = rel_l2(fin, ref_fin)
    say(f"  {label}: out max-abs {ea:.3e} (<= {out_tol:.3g}), "
        f"final rel-L2 {es:.3e} (<= {BF16_STATE_RELL2})")
    assert np.isfinite(out).all() and np.isfinite(fin).all()
    assert ea <= out_tol, f"{label}: output max-abs {ea}"
    assert es <= BF16_STATE_RELL2, f"{label}: final-state rel-L2 {es}"
    return ea, es


def check_f32(out, fin, ref_out, ref_fin, label=""):
    eo = rel_l2(out, ref_out)
    es = rel_l2(fin, ref_fin)
    say(f"  {label}: out rel-L2 {eo:.3e}, final rel-L2 {es:.3e} (<= {F32_RELL2})")
    assert eo <= F32_RELL2 and es <= F32_RELL2
    return eo, es


def need_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
