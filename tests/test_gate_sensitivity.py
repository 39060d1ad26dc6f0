"""The decay-gate GPU tests can see each plausible mistake (CPU, oracle only).

On the inputs of tests/test_gpu_f2.py's first decay case, the float64 oracle
is run with the reading's g and with g from a wrong reading of the flag: the
projection used as g itself (the flag ignored), the bias dropped, the rate
e^A replaced by A, or the rate ignored.  Each moves the outputs by far more
than the bf16 tolerance (2e-2 max-abs) the GPU test holds the kernels to, so
a kernel making that mistake fails it.
"""
import numpy as np

from gated_deltanet_02_amd import workloads as W
from oracle import gates, oracle

MUTANTS = {
    "flag ignored": lambda a, A, b: a,
    "bias dropped": lambda a, A, b: -np.exp(A) * gates.softplus(a),
    "rate not exponentiated": lambda a, A, b: -A * gates.softplus(a + b),
    "rate ignored": lambda a, A, b: -gates.softplus(a + b),
}


def test_decay_gate_mistakes_exceed_the_tolerance():
    w = W.make_workload("prompt_4k", lengths=[700], hk=2, hv=4)
    gi = W.make_gate_inputs(w)
    a, A, b = (x.numpy().astype(np.float64) for x in (gi.a, gi.a_log, gi.bias))
    ro, _ = oracle.reference(w.q, w.k, w.v, gates.decay_from_projection(a, A, b), w.beta,
                             w.lengths, w.init_state)
    for name, f in MUTANTS.items():
        with np.errstate(all="ignore"):
            mo, _ = oracle.reference(w.q, w.k, w.v, f(a, A, b), w.beta, w.lengths, w.init_state)
        err = np.abs(mo - ro)
        err = np.where(np.isfinite(err), err, np.inf).max()
        assert err > 10 * 2e-2, (name, err)
