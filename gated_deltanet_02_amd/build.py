"""Build the gfx950 library ``libgdn.so`` next to this file with hipcc.

Sources: csrc/gdn_kernels.hip (kernels, device code) and csrc/gdn_api.cpp
(the C ABI declared in include/gdn.h).  Compiled for gfx950 only, with packed
fp32 VALU instructions disabled.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgdn.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops: no packed fp32 arithmetic in the generated code.
# -amdgpu-mfma-vgpr-form: MFMA results in VGPRs, so accumulators that VALU
# code also updates (the scan's state) are not copied between the
# accumulator and vector register files.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          f"-I{INCLUDE}", f"-I{CSRC}"]
SOURCES = ["gdn_kernels.hip", "gdn_api.cpp"]


def build(verbose: bool = False) -> str:
    """Compile every source and link libgdn.so (always rebuilds)."""
    tmp = tempfile.mkdtemp(prefix="gdn_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            lang = ["-x", "hip"] if src.endswith(".hip") else []
            cmd = [HIPCC, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
            return obj
        with ThreadPoolExecutor(len(SOURCES)) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        out_tmp = LIB + ".tmp"
        cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed:\n{r.stderr}")
        os.replace(out_tmp, LIB)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
