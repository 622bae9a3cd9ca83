"""The public header compiles as C99 and a plain C program links against the
library and drives its host-side entry points (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

from residual_add_rmsnorm_rows_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_c_client_links_and_runs(tmp_path):
    if not os.path.exists(L.LIB_PATH):
        pytest.fail(f"{L.LIB_PATH} is not built")
    exe = tmp_path / "abi_check"
    libdir = os.path.dirname(L.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           f"-I{os.path.join(ROOT, 'include')}", os.path.join(ROOT, "tests", "c", "abi_check.c"),
           f"-L{libdir}", "-lrmsnorm_rows", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert "c abi check: ok" in out.stdout
