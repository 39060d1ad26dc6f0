"""Planted mistakes in the oracle must break at least one pin.

Each mutation edits one expression of oracle/gdn_oracle.c (a dropped term, a
wrong sign, a swapped operand or index), builds it into a temporary library
on the CPU, and runs the pins of tests/pins.py against it.  The mutated
library is never used for anything else.  All pins keep d_k = d_v where an
index swap is planted, so a mutated build stays in bounds.
"""
import os

import pytest

from oracle import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTATIONS = {
    "no_decay": ("*hij = alpha * (*hij - b * kh[i] * kTH[j])",
                 "*hij = (*hij - b * kh[i] * kTH[j])"),
    "erase_sign": ("(*hij - b * kh[i] * kTH[j])", "(*hij + b * kh[i] * kTH[j])"),
    "no_beta_on_write": ("+ b * kh[i] * (double)vt[j]", "+ kh[i] * (double)vt[j]"),
    "no_beta_on_erase": ("(*hij - b * kh[i] * kTH[j])", "(*hij - kh[i] * kTH[j])"),
    "decay_outside_write": ("*hij = alpha * (*hij - b * kh[i] * kTH[j]) + b * kh[i] * (double)vt[j];",
                            "*hij = alpha * ((*hij - b * kh[i] * kTH[j]) + b * kh[i] * (double)vt[j]);"),
    "transposed_state_read": ("kTH[j] += kh[i] * H[(size_t)i * dv + j]",
                              "kTH[j] += kh[i] * H[(size_t)j * dv + i]"),
    "output_reads_key": ("acc += H[(size_t)i * dv + j] * qh[i]",
                         "acc += H[(size_t)i * dv + j] * kh[i]"),
    "output_transposed": ("acc += H[(size_t)i * dv + j] * qh[i]",
                          "acc += H[(size_t)j * dv + i] * qh[i]"),
    "q_not_normalised": ("qh[i] = (double)qt[i] * rq;", "qh[i] = (double)qt[i];"),
    "k_not_normalised": ("kh[i] = (double)kt[i] * rk;", "kh[i] = (double)kt[i];"),
    "eps_outside_sqrt": ("1.0 / sqrt(kk + J->eps)", "1.0 / (sqrt(kk) + J->eps)"),
    "gate_not_exponentiated": ("const double alpha = exp((double)J->g",
                               "const double alpha = ((double)J->g"),
    "head_map_modulo": ("const int32_t kv = h / group;", "const int32_t kv = h % J->hk;"),
    "init_ignored": ("for (size_t e = 0; e < hsz; ++e) H[e] = (double)s[e];",
                     "for (size_t e = 0; e < hsz; ++e) H[e] = 0.0 * (double)s[e];"),
    "scale_dropped": ("ot[j] = J->scale * acc;", "ot[j] = acc;"),
    "skips_first_token": ("for (int32_t t = J->cu[seq]; t < J->cu[seq + 1]; ++t)",
                          "for (int32_t t = J->cu[seq] + 1; t < J->cu[seq + 1]; ++t)"),
    "output_before_update_uses_old_state": (
        "    /* kTH = k^T H  (a row of length dv) */",
        "    { double* o0 = J->out + ((size_t)t * J->hv + h) * dv;\n"
        "      for (int32_t j = 0; j < dv; ++j) { double a = 0.0;\n"
        "        for (int32_t i = 0; i < dk; ++i) a += H[(size_t)i * dv + j] * qh[i];\n"
        "        o0[j] = J->scale * a; } }\n"
        "    if (0) {\n"),
}


def _square_only(name):
    return name in ("transposed_state_read", "output_transposed")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mutated = src.replace(old, new, 1)
    if name == "output_before_update_uses_old_state":
        # close the 'if (0) {' opened above after the output block
        mutated = mutated.replace("      ot[j] = J->scale * acc;\n    }\n",
                                  "      ot[j] = J->scale * acc;\n    }\n    }\n", 1)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    lib_path = oracle.build(str(path), str(tmp_path / "libmut.so"))
    lib = oracle.load(lib_path)
    failed = []
    for pin, fn in pins.PINS.items():
        if _square_only(name) and pin == "brute_force":
            continue  # d_k != d_v there; an index swap would leave the buffer
        try:
            err = fn(lib)
        except ValueError:
            failed.append(pin)
            continue
        if not (err <= pins.PIN_TOL[pin]):  # also catches NaN
            failed.append(pin)
    assert failed, f"mutation {name} survived every pin"
