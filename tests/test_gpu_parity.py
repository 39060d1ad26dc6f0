"""HIP path vs the float64 oracle on the five workloads (GPU).

Reduced sizes and the full sizes alike compare every output and every final
state with the oracle.  The full sizes run the GPU exactly as the benchmark
does; the packed batch's oracle runs 32 sequences at a time to bound host
memory.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_02_amd import workloads as W
from oracle import oracle
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()
    oracle.load()


def _ref(w):
    return oracle.reference_workload(w)


REDUCED = [
    ("prompt_4k", dict(lengths=[1000], hk=4, hv=4)),
    ("long_16k_gqa", dict(lengths=[700], hk=2, hv=6)),
    ("packed_255", dict(lengths=("uniform", 12, 1, 300), hk=2, hv=2)),
    ("edge_mix", dict(hk=2, hv=2)),
    ("prompt_4k", dict(lengths=[333], hk=2, hv=2, dk=64, dv=64)),
    ("prompt_4k", dict(lengths=[257], hk=1, hv=2, dk=32, dv=128)),
    ("prompt_4k", dict(lengths=[77], hk=1, hv=1, dk=16, dv=16, chunk=16)),
    ("prompt_4k", dict(lengths=[190], hk=2, hv=4, dk=128, dv=64, chunk=32)),
    # 8 key heads with 2 value heads each: the one-slice scan places the
    # value heads of a key head on one XCD (a permuted head order)
    ("long_16k_gqa", dict(lengths=[260], hk=8, hv=16)),
]


# Enough (sequence, value head) pairs that 16-column slices would outnumber
# the compute units, so the scan runs two slices per workgroup; every output
# is checked.
GROUPED = [
    ("long_16k_gqa", dict(lengths=[300], hk=16, hv=48)),
    ("packed_255", dict(lengths=("uniform", 40, 1, 200), hk=8, hv=8)),
    ("prompt_4k", dict(lengths=[150] * 3, hk=12, hv=12, dk=64, dv=128)),
]


@pytest.mark.parametrize("name,kw", GROUPED, ids=[f"{n}-{i}" for i, (n, _) in enumerate(GROUPED)])
def test_reduced_two_slice_groups(name, kw):
    w = W.make_workload(name, **kw)
    heads = w.n_seqs * w.v.shape[1]
    assert heads * w.v.shape[2] // 16 > 256, "the case must queue one-slice workgroups"
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_bf16(out, fin, ro, rf, label=f"two-slice groups {name} {kw}")


# Enough (sequence, value head) pairs that four-slice workgroups still fill
# every compute unit, so the scan runs four slices per workgroup (two
# stages in its ring); every output is checked.
GROUPED4 = [
    ("packed_255", dict(lengths=("uniform", 140, 1, 200), hk=8, hv=8)),
    ("long_16k_gqa", dict(lengths=[200], hk=16, hv=128)),
    ("prompt_4k", dict(lengths=[150] * 3, hk=48, hv=48, dk=64, dv=128)),
    # small heads: the ring's stages are smaller, so it holds four of them
    ("packed_255", dict(lengths=("uniform", 64, 1, 150), hk=4, hv=4, dk=32, dv=64)),
    ("packed_255", dict(lengths=("uniform", 40, 1, 150), hk=2, hv=8, dk=16, dv=128)),
]


@pytest.mark.parametrize("name,kw", GROUPED4, ids=[f"{n}-{i}" for i, (n, _) in enumerate(GROUPED4)])
def test_reduced_four_slice_groups(name, kw):
    w = W.make_workload(name, **kw)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slices = w.n_seqs * w.v.shape[1] * w.v.shape[2] // 16
    assert slices >= 4 * cus, "the case must fill the compute units with four-slice workgroups"
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_bf16(out, fin, ro, rf, label=f"four-slice groups {name} {kw}")


@pytest.mark.parametrize("name,kw", REDUCED, ids=[f"{n}-{i}" for i, (n, _) in enumerate(REDUCED)])
def test_reduced_bf16(name, kw):
    w = W.make_workload(name, **kw)
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_bf16(out, fin, ro, rf, label=f"{name} {kw}")


def test_tiny_fp32_full():
    """Batch 1, T=64, 2 heads, d=16, chunk 16, fp32 inputs."""
    w = W.make_workload("tiny_fp32")
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_f32(out, fin, ro, rf, label="tiny_fp32")


@pytest.mark.parametrize("kw", [dict(lengths=[300], hk=2, hv=4, dk=64, dv=64, chunk=32),
                                dict(lengths=[45, 90, 1], hk=1, hv=2, dk=128, dv=32, chunk=16),
                                dict(lengths=[200], hk=1, hv=1, dk=128, dv=128, chunk=32,
                                     init_std=0.1)])
def test_fp32_more_shapes(kw):
    w = W.make_workload("tiny_fp32", **kw)
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_f32(out, fin, ro, rf, label=f"fp32 {kw}")


def test_prompt_4k_full():
    w = W.make_workload("prompt_4k")
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_bf16(out, fin, ro, rf, label="prompt_4k full")


def test_long_16k_gqa_full():
    """T=16384, 16 key heads shared by 48 value heads, random initial state:
    every output and the whole final state, with the oracle run once over
    all 48 (sequence, value head) units; also reported per key-head group."""
    w = W.make_workload("long_16k_gqa")
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    grp = w.v.shape[1] // w.q.shape[1]
    worst = 0.0
    for kh in range(w.q.shape[1]):
        hs = slice(kh * grp, (kh + 1) * grp)
        worst = max(worst, U.max_abs(out[:, hs], ro[:, hs]))
    U.say(f"  long_16k_gqa: worst key-head group out max-abs {worst:.3e}")
    U.check_bf16(out, fin, ro, rf, label="long_16k_gqa full")


def test_packed_255_full():
    """All 255 packed sequences: every output row and every final state,
    with the oracle run over runs of 32 consecutive sequences at a time
    (bounded host memory)."""
    w = W.make_workload("packed_255")
    U.say(f"  packed_255: T_total={w.t_total}")
    out, fin, _ = U.run_gpu(w)
    lens = np.asarray(w.lengths)
    starts = np.concatenate([[0], np.cumsum(lens)])
    worst_o, num, den = 0.0, 0.0, 0.0
    for a in range(0, len(lens), 32):
        idx = list(range(a, min(a + 32, len(lens))))
        sub = W.select_sequences(w, idx)
        ro, rf = _ref(sub)
        rows = slice(starts[idx[0]], starts[idx[-1] + 1])
        go, gf = out[rows], fin[idx[0]:idx[-1] + 1]
        U.check_bf16(go, gf, ro, rf, label=f"packed_255 sequences {idx[0]}-{idx[-1]}")
        worst_o = max(worst_o, U.max_abs(go, ro))
        num += float(np.sum((gf.astype(np.float64) - rf) ** 2))
        den += float(np.sum(rf ** 2))
    es = (num / den) ** 0.5
    U.say(f"  packed_255 whole batch: out max-abs {worst_o:.3e}, final rel-L2 {es:.3e}")
    assert worst_o <= U.BF16_OUT_MAXABS and es <= U.BF16_STATE_RELL2


def test_edge_mix_full_and_permuted():
    w = W.make_workload("edge_mix")
    out, fin, _ = U.run_gpu(w)
    ro, rf = _ref(w)
    U.check_bf16(out, fin, ro, rf, label="edge_mix")
    order = [3, 0, 4, 1, 2]  # lengths 65, 1, 1000, 63, 64
    wp = W.permute_sequences(w, order)
    assert wp.lengths == [65, 1, 1000, 63, 64]
    outp, finp, _ = U.run_gpu(wp)
    starts = np.concatenate([[0], np.cumsum(w.lengths)])
    startp = np.concatenate([[0], np.cumsum(wp.lengths)])
    for j, i in enumerate(order):
        # each sequence is computed by the same chunk arithmetic wherever it
        # sits in the batch: bitwise equal
        assert np.array_equal(outp[startp[j]:startp[j + 1]], out[starts[i]:starts[i + 1]])
        assert np.array_equal(finp[j], fin[i])
