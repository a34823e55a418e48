"""include/clo.h is a C header: a C11 caller (tests/c_header/use_clo.c, the
decode step as the README shows it) compiles with gcc under -pedantic with
warnings as errors, links against the built library and runs a host-only call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "top_sparse_attention_02_amd")


@pytest.mark.skipif(not shutil.which("gcc"), reason="needs gcc")
def test_header_compiles_as_c_and_links(tmp_path):
    from top_sparse_attention_02_amd import clo

    clo.load()  # the library is built
    exe = tmp_path / "use_clo"
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "c_header", "use_clo.c"), f"-L{LIBDIR}", "-lclo", f"-Wl,-rpath,{LIBDIR}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
