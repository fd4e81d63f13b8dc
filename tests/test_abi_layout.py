"""The ctypes mirrors in the Python binding against the C header: every
argument struct's size and every field's offset, as gcc lays them out for the
host (no GPU needed).  A field added to one side only fails here."""
import os
import subprocess
import tempfile

import pytest

import mamba_selective_scan_06_amd as ssm

STRUCTS = {
    "ssm_scan_args": ssm.ScanArgs,
    "ssm_scan_bwd_args": ssm.ScanBwdArgs,
    "ssm_conv_args": ssm.ConvArgs,
    "ssm_ssd_args": ssm.SsdArgs,
    "ssm_gla_args": ssm.GlaArgs,
}


@pytest.fixture(scope="module")
def c_layout():
    lines = ["#include <stddef.h>", "#include <stdio.h>", f'#include "{ssm.HEADER_PATH}"', "int main(void) {"]
    for cname, py in STRUCTS.items():
        lines.append(f'  printf("{cname} sizeof %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        with open(src, "w") as fh:
            fh.write("\n".join(lines) + "\n")
        subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", src, "-o", exe], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout
    table = {}
    for line in out.splitlines():
        s, f, v = line.split()
        table[(s, f)] = int(v)
    return table


@pytest.mark.parametrize("cname", sorted(STRUCTS))
def test_struct_layout_matches_header(cname, c_layout):
    py = STRUCTS[cname]
    assert c_layout[(cname, "sizeof")] == ctypes_sizeof(py), cname
    for f, _ in py._fields_:
        assert c_layout[(cname, f)] == getattr(py, f).offset, (cname, f)


def ctypes_sizeof(t):
    import ctypes
    return ctypes.sizeof(t)
