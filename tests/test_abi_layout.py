"""The C ABI's structs as C sees them against the Python binding (CPU).

include/gdn.h is compiled as C99 by gcc (no C++ in a C header), and a small
program prints the size of each struct the binding mirrors and the offset
of every field; the ctypes structures must agree field by field, so that
the options and layouts the binding passes are read as written.  The
header's status, dtype, stage, flag and scan constants must equal the
binding's.
"""
import ctypes
import os
import shutil
import subprocess

import pytest

from gated_deltanet_02_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {
    "gdn_tensor": B.GdnTensor,
    "gdn_options": B.GdnOptions,
    "gdn_workspace_layout": B.GdnWorkspaceLayout,
}


def c_layouts(tmp_path):
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "gdn.h"', "int main(void) {"]
    for name, cls in STRUCTS.items():
        lines.append(f'  printf("{name} size %zu\\n", sizeof({name}));')
        for field, _ in cls._fields_:
            lines.append(f'  printf("{name} {field} %zu\\n", offsetof({name}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", f"-I{ROOT}/include",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for line in out.splitlines():
        struct, key, value = line.split()
        got[(struct, key)] = int(value)
    return got


def test_binding_structs_match_the_c_header(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    got = c_layouts(tmp_path)
    for name, cls in STRUCTS.items():
        assert got[(name, "size")] == ctypes.sizeof(cls), name
        for field, _ in cls._fields_:
            assert got[(name, field)] == getattr(cls, field).offset, f"{name}.{field}"


def test_binding_constants_match_the_c_header():
    """Every status, dtype, stage, flag and scan constant the header
    defines has the same value in the binding."""
    import re
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    defs = {m.group(1): m.group(2) for m in re.finditer(r"^#define (GDN_\w+) (.+?)\s*(?:/\*.*)?$", src, re.M)}
    ints = {}
    for name, text in defs.items():
        m = re.fullmatch(r"\(?(-?\d+)u?\)?", text.strip())
        if m:
            ints[name] = int(m.group(1))
    expect = {
        "GDN_DTYPE_BF16": B._DTYPES[B.torch.bfloat16], "GDN_DTYPE_F32": B._DTYPES[B.torch.float32],
        "GDN_DTYPE_I32": B._DTYPES[B.torch.int32], "GDN_DTYPE_I64": B._DTYPES[B.torch.int64],
        "GDN_STAGE_TABLE": B.STAGE_TABLE, "GDN_STAGE_WY": B.STAGE_WY, "GDN_STAGE_SCAN": B.STAGE_SCAN,
        "GDN_STAGE_ALL": B.STAGE_ALL,
        "GDN_SCAN_AUTO": B.SCAN_AUTO, "GDN_SCAN_ONE_PASS": B.SCAN_ONE_PASS,
        "GDN_SCAN_TWO_LEVEL": B.SCAN_TWO_LEVEL,
        "GDN_FLAG_BETA_LOGITS": B.FLAG_BETA_LOGITS, "GDN_FLAG_DECAY_PROJ": B.FLAG_DECAY_PROJ,
        "GDN_FLAG_OUTPUT_GATE": B.FLAG_OUTPUT_GATE, "GDN_FLAG_QKV_SILU": B.FLAG_QKV_SILU,
        "GDN_FLAG_QKV_CONV": B.FLAG_QKV_CONV,
    }
    for name, value in B.STATUS_NAMES.items():
        expect[value] = name
    for name, value in expect.items():
        assert ints[name] == value, name
    # every flag, stage and scan constant of the header is covered
    for name in ints:
        if name.startswith(("GDN_FLAG_", "GDN_STAGE_", "GDN_SCAN_", "GDN_ERR_", "GDN_DTYPE_")):
            assert name in expect, f"{name} has no binding constant"
    assert ints["GDN_OK"] == 0 and B.GDN_OK == 0
    assert B.NOALLOC_SCRATCH_BYTES == 96 << 20 and "((size_t)96 << 20)" in defs["GDN_NOALLOC_SCRATCH_BYTES"]


def test_binding_abi_version_and_missing_library():
    """The binding states the header's ABI version, and it refuses a missing
    library with a clear error instead of running anything else."""
    import re
    import sys
    src = open(os.path.join(ROOT, "include", "gdn.h")).read()
    assert B.ABI_VERSION == int(re.search(r"#define GDN_ABI_VERSION (\d+)", src).group(1))
    code = ("import gated_deltanet_02_amd as G\n"
            "try:\n    G.gdn_abi_version()\nexcept RuntimeError as e:\n    print('refused:', e)\n")
    env = dict(os.environ, GDN_LIB="/nonexistent/libgdn.so")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=120)
    assert r.returncode == 0 and "refused: libgdn.so not found" in r.stdout, r.stdout + r.stderr


def test_binding_refuses_another_abi(tmp_path):
    """A library that reports another ABI version (a stand-in built here that
    exports only gdn_abi_version) is refused at load."""
    import sys
    if not shutil.which("gcc"):
        pytest.skip("gcc not found")
    src = tmp_path / "old.c"
    src.write_text(f"int gdn_abi_version(void) {{ return {B.ABI_VERSION - 1}; }}\n")
    so = tmp_path / "libold.so"
    subprocess.run(["gcc", "-shared", "-fPIC", str(src), "-o", str(so)], check=True)
    code = ("import gated_deltanet_02_amd as G\n"
            "try:\n    G.gdn_abi_version()\nexcept RuntimeError as e:\n    print('refused:', e)\n")
    env = dict(os.environ, GDN_LIB=str(so))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=120)
    assert r.returncode == 0 and f"implements ABI {B.ABI_VERSION - 1}" in r.stdout, r.stdout + r.stderr
