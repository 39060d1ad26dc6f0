"""The C ABI's structs as C sees them against the Python binding (CPU).

include/gdn.h is compiled as C99 by gcc (no C++ in a C header), and a small
program prints the size of each struct the binding mirrors and the offset
of every field; the ctypes structures must agree field by field, so that
the options and layouts the binding passes are read as written.
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
