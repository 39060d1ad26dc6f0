"""bench.py's contract, on the CPU: one GPU only, and the algorithmic bytes
and flops its roofline divides by, against the per-token figures worked out
from the shapes by hand."""
import os
import subprocess
import sys

import bench
from gated_deltanet_02_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_of_the_4096_token_prompt():
    w = W.make_workload("prompt_4k")
    # per token: q and k (16 heads x 128, bf16), v and out (16 x 128, bf16),
    # g and beta (16 fp32 each): 8192 + 8192 + 128 = 16,512 bytes; plus the
    # fp32 final state 16 x 128 x 128 x 4 (no initial state is read)
    assert bench.algorithmic_bytes(w) == 4096 * 16512 + 16 * 128 * 128 * 4 == 68_681_728


def test_algorithmic_bytes_count_the_initial_state_when_given():
    w = W.make_workload("long_16k_gqa", lengths=[100], hk=2, hv=6, dk=32, dv=16)
    per_token = 2 * 2 * 32 * 2 + 2 * 6 * 16 * 2 + 2 * 6 * 4
    assert w.init_state is not None
    assert bench.algorithmic_bytes(w) == 100 * per_token + 2 * 6 * 32 * 16 * 4


def test_algorithmic_flops_of_the_4096_token_prompt():
    w = W.make_workload("prompt_4k")
    # per value-head token at C = 64, d = 128: 63*128 + 65*128 + 64^2/3 +
    # 65*256 + 6*128^2 + 65*128 = 141,013.33
    per = 63 * 128 + 65 * 128 + 64 * 64 / 3 + 65 * 256 + 6 * 128 * 128 + 65 * 128
    assert abs(per - 141013.33) < 0.01
    assert bench.algorithmic_flops(w) == int(4096 * 16 * per)
