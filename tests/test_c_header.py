"""The boundary from C: include/moe_route.h compiles as strict C99 and as
C++17, and a C program built against it links with the library and gets
the documented host-side answers (status strings, workspace sizes,
argument rejection before any launch). No GPU is touched."""
import os
import shutil
import subprocess
import tempfile

import pytest

from permutation_group_limited_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

PROGRAM = r"""
#include <stdio.h>
#include "moe_route.h"

int main(void) {
  int32_t idx[8];
  float w[8], s[64], b[8];
  printf("%s\n", moe_status_string(MOE_ERR_INVALID_ARG));
  printf("%zu\n", moe_create_indices_workspace_size(1024, 256));
  printf("%zu\n", moe_create_indices_workspace_size(65536, 256));
  printf("%zu\n", moe_route_and_index_workspace_size(128, 8, 256));
  /* T < 0: rejected on the host, nothing launched */
  printf("%d\n", (int)moe_router_group_limited(idx, w, s, b, MOE_DTYPE_F32, MOE_DTYPE_F32, -1,
                                                8, 2, 1, 1, 1, 1.0f, MOE_GROUP_TOP2_SUM, NULL));
  return 0;
}
"""


def _cc():
    return shutil.which("gcc")


@pytest.mark.skipif(_cc() is None, reason="no C compiler")
@pytest.mark.parametrize("header", ["moe_route.h", "moe_probe.h"])
@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_compiles(lang, std, header):
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "h." + ("c" if lang == "c" else "cc"))
        with open(src, "w") as f:
            f.write('#include "%s"\n' % header)
        r = subprocess.run([_cc(), "-x", lang, std, "-Wall", "-Wextra", "-Werror", "-pedantic",
                            "-fsyntax-only", "-I", INCLUDE, src], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


@pytest.mark.skipif(_cc() is None, reason="no C compiler")
def test_c_program_links_and_validates():
    lib = binding.library_path()
    if not os.path.exists(lib):
        from permutation_group_limited_amd import build
        build.build()
    libdir = os.path.dirname(lib)
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        with open(src, "w") as f:
            f.write(PROGRAM)
        r = subprocess.run([_cc(), "-std=c99", "-Wall", "-Werror", "-I", INCLUDE, src, "-o", exe,
                            lib, "-Wl,-rpath," + libdir], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        assert r.returncode == 0, r.stderr
        lines = r.stdout.split()
    expect_ws = binding.moe_create_indices_workspace_size(65536, 256)
    expect_ri = binding.moe_route_and_index_workspace_size(128, 8, 256)
    assert lines[-4:] == ["0", str(expect_ws), str(expect_ri), "1"]
    assert "INVALID" in r.stdout.upper()
