"""The binding's ctypes structs against the C layout of include/halo.h: a small C program,
compiled with the host compiler against the header, prints every field's offset and each
struct's size, and the ctypes definitions must match them field by field (CPU only)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import hadamard_rotated_precision_halo_amd as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

STRUCTS = {"halo_quant_opts": H.QuantOpts, "halo_linear_opts": H.LinearOpts}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs the host C compiler")
def test_opts_structs_match_the_header(tmp_path):
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "halo.h"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    c = {(a, b): int(v) for a, b, v in (l.split() for l in out if l)}
    for cname, py in STRUCTS.items():
        assert c[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert c[(cname, field)] == getattr(py, field).offset, (cname, field)


def test_header_declares_no_other_opts_fields():
    # every field the header gives the two structs is one the binding passes, in order
    text = open(os.path.join(ROOT, "include", "halo.h")).read()
    for cname, py in STRUCTS.items():
        body = re.search(r"typedef struct \{([^{}]*)\} " + cname + ";", text).group(1)
        body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
        names = re.findall(r"(\w+)\s*(?:\[\d+\])?\s*;", body)
        assert names == [f for f, _ in py._fields_], cname
