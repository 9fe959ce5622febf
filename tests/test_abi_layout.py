"""The binding's ctypes structs lay out exactly like the C header's: every
field at the same offset with the same size, and the same total size
(checked with gcc against include/aggemm.h; no GPU needed)."""
import ctypes
import os
import shutil
import subprocess

import pytest

from communication_gemm_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc needed")


def c_layout(tmp_path, struct, fields):
    lines = [f'printf("%zu\\n", sizeof({struct}));']
    for f in fields:
        lines.append(f'printf("%zu %zu\\n", offsetof({struct}, {f}), sizeof((({struct} *)0)->{f}));')
    src = tmp_path / f"{struct}.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "aggemm.h"\n'
                   'int main(void) {\n' + "\n".join(lines) + "\nreturn 0;\n}\n")
    exe = tmp_path / struct
    subprocess.run(["gcc", "-std=c11", f"-I{os.path.join(ROOT, 'include')}", str(src), "-o",
                    str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    size = int(out[0])
    return size, [tuple(int(x) for x in line.split()) for line in out[1:1 + len(fields)]]


@pytest.mark.parametrize("struct,cls", [("agg_options", _native.Options),
                                        ("agg_plan_info", _native.PlanInfo)])
def test_struct_layout_matches_header(tmp_path, struct, cls):
    names = [f for f, _ in cls._fields_]
    size, layout = c_layout(tmp_path, struct, names)
    assert size == ctypes.sizeof(cls), (struct, size, ctypes.sizeof(cls))
    for name, (off, sz) in zip(names, layout):
        field = getattr(cls, name)
        assert (field.offset, field.size) == (off, sz), (struct, name, off, sz)
