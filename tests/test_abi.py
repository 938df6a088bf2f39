"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/svt.h declares, and the Python binding's argument
structs match the header's field order, types and byte layout."""
import ctypes
import os
import re
import subprocess

import pytest

from tree_masked_verification_parent_amd import svt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svt.h")


def _header():
    with open(HEADER) as f:
        return f.read()


def _declared_functions(text):
    return re.findall(r"^[A-Za-z][\w \*]*?\b(svt_\w+)\(", text, flags=re.M)


def _structs(text):
    """{name: [(c_type, field), ...]} for the typedef'd argument structs."""
    out = {}
    for m in re.finditer(r"typedef struct (svt_\w+) \{(.*?)\} \1;", text, flags=re.S):
        body = re.sub(r"/\*.*?\*/", "", m.group(2), flags=re.S)
        fields = []
        for decl in body.split(";"):
            decl = decl.strip()
            if not decl:
                continue
            ctype, names = re.match(r"((?:const\s+)?[\w]+\s*\**)\s*(.*)", decl).groups()
            for n in names.split(","):
                n = n.strip()
                stars = n.count("*")
                fields.append((ctype.replace(" ", "") + "*" * stars, n.strip("* ")))
        out[m.group(1)] = fields
    return out


def test_library_exports_every_declared_function():
    lib = svt.lib()
    declared = _declared_functions(_header())
    assert set(declared) == set(svt.EXPORTS), (sorted(declared), sorted(svt.EXPORTS))
    for name in declared:
        assert hasattr(lib, name), name


def test_version_and_status_strings_without_gpu():
    lib = svt.lib()
    lib.svt_version.restype = ctypes.c_char_p
    assert b"gfx950" in lib.svt_version()
    lib.svt_status_string.restype = ctypes.c_char_p
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9]:
        assert lib.svt_status_string(code)
    assert lib.svt_status_string(0) != lib.svt_status_string(-1)


_C_TO_CTYPES = {
    "int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "float": ctypes.c_float, "size_t": ctypes.c_size_t,
}


STRUCTS = [("svt_attn_args", "AttnArgs"), ("svt_accept_args", "AcceptArgs"), ("svt_commit_args", "CommitArgs"),
           ("svt_realign_args", "RealignArgs")]


@pytest.mark.parametrize("cname,pyname", STRUCTS)
def test_binding_structs_match_header(cname, pyname):
    fields = _structs(_header())[cname]
    py = getattr(svt, pyname)._fields_
    assert [f for _, f in fields] == [n for n, _ in py]
    for (ctype, name), (_, pytype) in zip(fields, py):
        if ctype.endswith("*"):
            assert pytype is ctypes.c_void_p, name
        else:
            base = ctype.replace("const", "")
            assert ctypes.sizeof(pytype) == ctypes.sizeof(_C_TO_CTYPES[base]), name


def test_struct_sizes_match_the_c_compiler(tmp_path):
    """sizeof and offsetof of every field, from a host C compile of the header."""
    text = _header()
    structs = _structs(text)
    src = ["#include <stdio.h>", "#include <stddef.h>", '#include "svt.h"', "int main(void) {"]
    for cname, _ in STRUCTS:
        src.append(f'  printf("{cname} %zu\\n", sizeof({cname}));')
        for _, f in structs[cname]:
            src.append(f'  printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    src.append("  return 0;\n}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(src))
    exe = tmp_path / "layout"
    cmd = ["gcc", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I",
           "/opt/rocm/include", str(c), "-o", str(exe)]
    try:
        subprocess.run(cmd, check=True, capture_output=True)
    except (OSError, subprocess.CalledProcessError) as e:
        pytest.skip(f"host compile of svt.h unavailable: {e}")
    got = dict(line.rsplit(" ", 1) for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                              check=True).stdout.split("\n") if line)
    for cname, pyname in STRUCTS:
        py = getattr(svt, pyname)
        assert int(got[cname]) == ctypes.sizeof(py), cname
        for _, f in structs[cname]:
            assert int(got[f"{cname}.{f}"]) == getattr(py, f).offset, (cname, f)
