"""Seeded synthetic inputs: reproducible, right shapes, right distributions."""
import numpy as np
import torch

from gated_deltanet_02_amd import workloads as W


def test_reproducible_bitwise():
    a = W.make_workload("edge_mix")
    b = W.make_workload("edge_mix")
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.g, b.g), (a.beta, b.beta)]:
        assert torch.equal(x, y)
    c = W.make_workload("edge_mix", seed=1)
    assert not torch.equal(a.q, c.q)


def test_shapes_and_dtypes():
    w = W.make_workload("tiny_fp32")
    assert w.q.shape == (64, 2, 16) and w.q.dtype == torch.float32
    assert w.chunk == 16 and w.init_state is None
    w = W.make_workload("prompt_4k", lengths=[256])
    assert w.q.dtype == torch.bfloat16 and w.v.shape == (256, 16, 128)
    w = W.make_workload("long_16k_gqa", lengths=[128], hk=2, hv=6)
    assert w.init_state.shape == (1, 6, 128, 128)
    w = W.make_workload("edge_mix")
    assert w.lengths == [1, 63, 64, 65, 1000] and w.t_total == 1193
    assert w.cu_seqlens.tolist() == [0, 1, 64, 128, 193, 1193]
    assert w.token_offset == 1


def test_packed_lengths_range():
    r = np.random.default_rng(0)
    lens = r.integers(200, 4097, size=255)
    w = W.make_workload("packed_255", hk=1, hv=1, dk=16, dv=16)
    assert w.lengths == [int(x) for x in lens]
    assert min(w.lengths) >= 200 and max(w.lengths) <= 4096


def test_distributions():
    w = W.make_workload("prompt_4k", lengths=[2048], hk=4, hv=4)
    qn = w.q.float().norm(dim=-1)
    assert torch.allclose(qn, torch.ones_like(qn), atol=1e-2)   # unit rows, bf16
    assert -1.0 <= float(w.g.min()) and float(w.g.max()) <= 0.0
    assert abs(float(w.g.mean()) + 0.5) < 0.02
    assert abs(float(w.v.float().std()) - 1.0) < 0.02
    b = w.beta.double()
    assert 0.0 < float(b.min()) and float(b.max()) < 1.0
    assert abs(float(b.mean()) - 0.5) < 0.01
    w = W.make_workload("long_16k_gqa", lengths=[64], hk=1, hv=3)
    assert abs(float(w.init_state.std()) - 0.1) < 0.005


def test_edge_mix_classes():
    w = W.make_workload("edge_mix")
    g = w.g.numpy()
    zero_rows = np.all(g == 0.0, axis=1)
    assert zero_rows.sum() == round(0.25 * w.t_total)
    assert g.min() >= -8.0
    b = w.beta.numpy()
    lo = np.isclose(b, 1 / (1 + np.exp(12.0)), rtol=1e-6)
    hi = np.isclose(b, 1 / (1 + np.exp(-12.0)), rtol=1e-7)
    assert 0.28 < lo.mean() < 0.39 and 0.28 < hi.mean() < 0.39


def test_permute_and_select_are_data_movement():
    w = W.make_workload("edge_mix", hk=1, hv=1, dk=16, dv=16)
    p = W.permute_sequences(w, [3, 0, 4, 2, 1])
    assert p.lengths == [65, 1, 1000, 64, 63]
    assert torch.equal(p.q[:65], w.q[128:193])
    s = W.select_sequences(w, [4])
    assert torch.equal(s.v, w.v[193:])
