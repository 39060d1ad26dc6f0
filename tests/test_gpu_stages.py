"""Each stage's intermediates vs the float64 chunked evaluator (GPU).

The chunk table and the WY stage run alone on a caller-owned workspace; the
per-(chunk, value head) blocks are then read back through the documented
workspace layout and compared with oracle/chunked.py's intermediates.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_02_amd as G
from gated_deltanet_02_amd import workloads as W
from oracle import chunked
from tests import gpu_util as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    U.need_gpu()


def _blocks(ws, off, count, shape, dtype):
    n = int(np.prod(shape)) * count
    es = torch.tensor([], dtype=dtype).element_size()
    return ws[off:off + n * es].view(dtype).view(count, *shape).float().cpu().numpy()


def ktile_pos(K, m, k, two_byte):
    """Position of element (m, k) of a 16 x K tile stored in k-tile order:
    for the 16-wide k-tile t = k // 16, lane m + 16 ((k % 16) // 4) holds
    the four elements k % 4 = 0..3.  Two-byte types pair k-tiles (2u, 2u+1)
    into one 8-element unit per lane (a trailing single k-tile: 4 elements);
    fp32 has one k-tile per unit."""
    t, g, e = k // 16, (k % 16) // 4, k % 4
    lane = m + 16 * g
    if not two_byte:
        return t * 256 + lane * 4 + e
    nt = K // 16
    u, h = t // 2, t % 2
    half_tail = (nt % 2 == 1) & (u == nt // 2)
    return np.where(half_tail, u * 512 + lane * 4 + e, u * 512 + lane * 8 + 4 * h + e)


def unfrag(blocks, rows, K, two_byte):
    """[count, rows*K] in k-tile order (16-row tiles) -> [count, rows, K]."""
    r = np.arange(rows)[:, None]
    k = np.arange(K)[None, :]
    idx = (r // 16) * 16 * K + ktile_pos(K, r % 16, k, two_byte)
    return blocks.reshape(blocks.shape[0], -1)[:, idx]


def unacc(blocks, rows, cols, transposed):
    """Accumulator-layout tiles ([tile][lane][4]) -> dense [count, rows, cols],
    tiles column-tile major: tile (ct, rt) = ct * (rows/16) + rt.  Not
    transposed: lane l holds rows 4 (l/16) + e, column l % 16.  Transposed
    (O^T tiles): lane l holds columns 4 (l/16) + e of row l % 16."""
    r = np.arange(rows)[:, None]
    c = np.arange(cols)[None, :]
    if not transposed:
        tile = (c // 16) * (rows // 16) + r // 16
        lane = (c % 16) + 16 * ((r % 16) // 4)
        e = (r % 16) % 4
    else:
        tile = (c // 16) * (rows // 16) + r // 16
        lane = (r % 16) + 16 * ((c % 16) // 4)
        e = (c % 16) % 4
    idx = tile * 256 + lane * 4 + e
    return blocks.reshape(blocks.shape[0], -1)[:, idx]


CASES = [
    ("bf16-single", "prompt_4k", dict(lengths=[150], hk=2, hv=4, dk=64, dv=64), 2e-2),
    ("bf16-packed", "edge_mix", dict(lengths=[70, 1, 64, 30, 0, 129], hk=1, hv=2, dk=128, dv=128), 2e-2),
    ("bf16-c32", "prompt_4k", dict(lengths=[100], hk=1, hv=1, dk=32, dv=64, chunk=32), 2e-2),
    ("f32-c16", "tiny_fp32", dict(lengths=[64, 7], hk=2, hv=2), 2e-6),
    ("f32-c32", "tiny_fp32", dict(lengths=[75], hk=1, hv=3, dk=128, dv=32, chunk=32), 2e-6),
]


@pytest.mark.parametrize("label,name,kw,tol", CASES, ids=[c[0] for c in CASES])
def test_wy_intermediates(label, name, kw, tol):
    w = W.make_workload(name, **kw)
    d = W.to_device(w)
    C = w.chunk
    cu = d["cu_seqlens"] if w.n_seqs > 1 else None
    opts = G.options(chunk=C, stages=G.STAGE_TABLE | G.STAGE_WY)
    lay = G.gdn_get_workspace_layout(d["q"], d["k"], d["v"], cu, opts)
    ws = torch.zeros(lay.total_bytes, dtype=torch.uint8, device="cuda")
    U.say(f"  {label}: stages table+wy, max_chunks={lay.max_chunks}")
    G.gdn_prefill_ex(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, d["init_state"],
                     d["out"], d["final_state"], opts=opts, workspace=ws)
    torch.cuda.synchronize()
    keep = []
    chunked.chunked_reference(w.q, w.k, w.v, w.g, w.beta, w.lengths, w.init_state,
                              chunk=C, keep=keep)
    hv, dk, dv = w.v.shape[1], w.q.shape[2], w.v.shape[2]
    mc = lay.max_chunks
    dt = w.q.dtype
    two = dt == torch.bfloat16
    Wb = unfrag(_blocks(ws, lay.w, mc * hv, (C, dk), dt), C, dk, two)
    Qp = unfrag(_blocks(ws, lay.qp, mc * hv, (C, dk), dt), C, dk, two)
    Ut = np.swapaxes(unacc(_blocks(ws, lay.ut, mc * hv, (C, dv), dt), C, dv, False), 1, 2)
    Ol = unacc(_blocks(ws, lay.oloc, mc * hv, (C, dv), dt), C, dv, True)
    dec = _blocks(ws, lay.decay, mc * hv, (1,), torch.float32)[:, 0]
    if w.n_seqs > 1:
        table = _blocks(ws, lay.chunk_table, mc, (4,), torch.int32).astype(np.int64)
    nchunks = [-(-L // C) for L in w.lengths]
    first = np.concatenate([[0], np.cumsum(nchunks)])
    starts = np.concatenate([[0], np.cumsum(w.lengths)])

    def close(a, b, what):
        scale_ = max(float(np.abs(b).max()), 1e-30)
        err = float(np.abs(a - b).max()) / scale_
        assert err <= tol, f"{label} {what}: relative error {err:.3e} > {tol}"
        return err

    worst = {}
    for it in keep:
        c = int(first[it["seq"]] + it["chunk"])
        n = it["n"]
        blk = c * hv + it["head"]
        if w.n_seqs > 1:
            assert table[c, 0] == it["seq"] and table[c, 1] == it["t0"] and table[c, 2] == n
            assert it["t0"] == starts[it["seq"]] + it["chunk"] * C
        # W and U~ are stored with row r scaled by s_r = e^(gamma_last - gamma_r)
        # / sqrt(|k_r|^2 + eps) (k_r the key row as passed), so that the scan's
        # state update can take the key rows as they are
        kh_ = it["head"] // (hv // w.q.shape[1])
        kr = w.k[it["t0"]:it["t0"] + n, kh_].double().numpy()
        s = np.exp(it["gamma"][-1] - it["gamma"]) / np.sqrt((kr * kr).sum(-1) + 1e-6)
        for what, got, ref in (("W", Wb[blk, :n], s[:, None] * it["W"]),
                               ("Qprime", Qp[blk, :n], it["Qprime"]),
                               ("Utilde^T", Ut[blk][:, :n], (s[:, None] * it["Utilde"]).T),
                               ("Oloc", Ol[blk, :n], it["Oloc"])):
            worst[what] = max(worst.get(what, 0.0), close(got, ref, what))
        # the scaled rows are the key rows the state update meets: K~ = diag(s) K
        assert np.allclose(s[:, None] * kr, it["Ktilde"], rtol=1e-6, atol=1e-9)
        # rows past the chunk's end are zero
        assert not Wb[blk, n:].any() and not Qp[blk, n:].any()
        assert not Ut[blk][:, n:].any() and not Ol[blk, n:].any()
        assert abs(dec[blk] - np.exp(it["gamma"][-1])) <= 1e-5 * max(1.0, np.exp(it["gamma"][-1]))
    U.say(f"  {label}: worst relative errors {worst}")
