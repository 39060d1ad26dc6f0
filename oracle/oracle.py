"""Python entry to the float64 Gated DeltaNet reference -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module.  It builds ``oracle/liboracle.so`` from
``gdn_oracle.c`` with the host C compiler and calls it through ctypes.  It
imports nothing from the HIP package.

The recurrence and its citation are in the header of ``gdn_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags: Sequence[str] = ()) -> str:
    """Compile the reference with plain -O2 (no fast-math: every product and
    sum is evaluated in the written order)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: Optional[str] = None):
    """Load (building first if needed) the reference library."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if (not os.path.exists(_LIB)
                or os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        path = _LIB
    lib = ctypes.CDLL(path)
    f = lib.gdn_oracle_f64
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    f.argtypes = [P, P, P, P, P, P, i32, P, P, P, i32, i32, i32, i32, i32,
                  ctypes.c_double, ctypes.c_double, i32]
    f.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _f32(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (bf16 values are exact in float32)
        x = x.detach().to("cpu").float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def reference(q, k, v, g, beta, lengths: Sequence[int], init_state=None,
              scale: float = 1.0, eps: float = 1e-6, want_final: bool = True,
              threads: int = 0, lib=None):
    """Token-by-token float64 Gated DeltaNet over packed sequences.

    q, k: [T, Hk, dk]; v: [T, Hv, dv]; g, beta: [T, Hv]; ``lengths`` the
    per-sequence token counts (packed in order); init_state [N, Hv, dk, dv]
    or None (zeros).  Returns (out [T, Hv, dv], final [N, Hv, dk, dv] or
    None) as float64 numpy arrays.
    """
    q, k, v, g, beta = (_f32(a) for a in (q, k, v, g, beta))
    init = _f32(init_state)
    T, hk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    n = len(lengths)
    cu = np.zeros(n + 1, np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    if cu[-1] != T:
        raise ValueError("lengths do not sum to T")
    out = np.empty((T, hv, dv), np.float64)
    final = np.empty((n, hv, dk, dv), np.float64) if want_final else None
    lib = lib or load()
    ptr = lambda a: None if a is None else a.ctypes.data  # noqa: E731
    rc = lib.gdn_oracle_f64(ptr(q), ptr(k), ptr(v), ptr(g), ptr(beta),
                            ptr(cu), n, ptr(init), ptr(out), ptr(final),
                            T, hk, hv, dk, dv, float(scale), float(eps),
                            int(threads))
    if rc != 0:
        raise ValueError(f"oracle rejected its arguments (rc={rc})")
    return out, final


def reference_workload(w, scale: float = 1.0, eps: float = 1e-6,
                       threads: int = 0, lib=None):
    """``reference`` on a ``Workload`` from the seeded input module."""
    return reference(w.q, w.k, w.v, w.g, w.beta, w.lengths, w.init_state,
                     scale=scale, eps=eps, threads=threads, lib=lib)
