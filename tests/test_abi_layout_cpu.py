"""The ctypes mirrors of the C-ABI structs match include/lcx.h field for field:
a small C program built with gcc against the header prints every field's
offset and each struct's size, and the binding's ctypes structures must agree
(a mismatch would hand the library misplaced arguments without any error)."""
import ctypes
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcx.h")


def _c_layout(tmp_path, structs):
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "lcx.h"', "int main(void) {"]
    for cname, fields in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f in fields:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run(["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                        "-I", "/opt/rocm/include", str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for line in out.splitlines():
        cname, key, val = line.split()
        got[(cname, key)] = int(val)
    return got


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_ctypes_structs_match_the_header(tmp_path):
    import long_context_attention_rope_amd as lcx
    pairs = {"lcx_rope_cfg": lcx.RopeCfg, "lcx_attn_args": lcx.AttnArgs, "lcx_attn_bwd_args": lcx.BwdArgs}
    structs = {c: [f[0] for f in t._fields_] for c, t in pairs.items()}
    got = _c_layout(tmp_path, structs)
    for cname, t in pairs.items():
        assert got[(cname, "size")] == ctypes.sizeof(t), cname
        for f in structs[cname]:
            assert got[(cname, f)] == getattr(t, f).offset, (cname, f)
