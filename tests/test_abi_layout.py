"""The Python binding's ctypes structs against the C header's layout.

The binding mirrors each argument struct of include/hswa.h by hand; a field
out of order, a wrong width or a missing field would hand the library
garbage without any error.  This compiles a small C program against the
header with the host C compiler, prints sizeof and offsetof of every field
of every struct, and requires the ctypes mirror to agree field by field
(same names, same order, same offsets, same total size).
"""
import ctypes as C
import os
import re
import shutil
import subprocess

import pytest

from hybrid_sliding_window_hswa_amd import _capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# C struct name -> ctypes mirror
STRUCTS = {
    "hswa_pool_desc": _capi.PoolDesc,
    "hswa_pool_view": _capi.PoolView,
    "hswa_attn_args": _capi.AttnArgs,
    "hswa_xfer_args": _capi.XferArgs,
    "hswa_kv_copy_args": _capi.KvCopyArgs,
}


def _c_layout(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    lines = ['#include <stddef.h>', '#include <stdio.h>', '#include "hswa.h"', 'int main(void) {']
    for cname, mirror in STRUCTS.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for fname, _ in mirror._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    r = subprocess.run([cc, "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr    # a mirror field the header lacks fails here
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    got = {}
    for line in out.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    return got


def _c_fields(cname):
    """Field names of a struct in include/hswa.h, in declaration order."""
    with open(os.path.join(ROOT, "include", "hswa.h")) as f:
        text = f.read()
    body = text[text.index(f"typedef struct {cname} {{"):]
    body = body[body.index("{") + 1:body.index(f"}} {cname};")]
    body = re.sub(r"/\*.*?\*/", " ", body, flags=re.S)   # comments may hold ';'
    names = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            names.append(decl.replace("*", " ").split()[-1])
    return names


@pytest.mark.parametrize("cname", sorted(STRUCTS))
def test_ctypes_mirror_matches_header(cname, tmp_path):
    mirror = STRUCTS[cname]
    assert [f for f, _ in mirror._fields_] == _c_fields(cname), "field names or order"
    got = _c_layout(tmp_path)
    assert got[(cname, "sizeof")] == C.sizeof(mirror)
    for fname, _ in mirror._fields_:
        assert got[(cname, fname)] == getattr(mirror, fname).offset, fname
