"""The library's host code (selector, argument checks, C ABI) under
AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

select.cpp and abi.cpp are rebuilt with g++ ``-fsanitize=address,undefined``
(host code only: the kernel objects are linked as built), then two C clients
run against them: ``tests/c/abi_check.c`` and ``tests/c/fuzz_host.c``, a
randomized sweep of 200,000 query and argument-check calls whose explicit
launch configurations are always rejected, so nothing reaches a kernel
launch.  Any sanitizer report fails the test.
"""

from __future__ import annotations

import os
import shutil
import subprocess

import pytest

from residual_add_rmsnorm_rows_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="gcc / g++ not found")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    kernel_objs = [obj for obj, cmd in B._jobs() if any(a.endswith(".hip") for a in cmd)]
    missing = [o for o in kernel_objs if not os.path.exists(o)]
    if missing:
        pytest.fail(f"kernel objects not built (run the build first): {missing[:3]}")
    d = tmp_path_factory.mktemp("san")
    host = ["-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{B.ROCM}/include", f"-I{B.INCLUDE}", f"-I{B.CSRC}"]
    objs = []
    for src in ("select.cpp", "abi.cpp"):
        o = str(d / src.replace(".cpp", ".o"))
        subprocess.run(["g++", *host, *SAN, "-c", os.path.join(B.CSRC, src), "-o", o], check=True,
                       capture_output=True, text=True)
        objs.append(o)
    exes = {}
    for name in ("abi_check", "fuzz_host"):
        o = str(d / f"{name}.o")
        subprocess.run(["gcc", "-std=c99", *SAN, f"-I{B.INCLUDE}", "-c",
                        os.path.join(ROOT, "tests", "c", f"{name}.c"), "-o", o], check=True, capture_output=True,
                       text=True)
        exe = str(d / name)
        subprocess.run(["g++", *SAN, o, *objs, *kernel_objs, f"-L{B.ROCM}/lib", "-lamdhip64",
                        f"-Wl,-rpath,{B.ROCM}/lib", "-o", exe], check=True, capture_output=True, text=True)
        exes[name] = exe
    return exes


@pytest.mark.parametrize("name,expect", [("abi_check", "c abi check: ok"), ("fuzz_host", "fuzz ok")])
def test_clients_run_clean_under_sanitizers(sanitized, name, expect):
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    out = subprocess.run([sanitized[name]], capture_output=True, text=True, timeout=600, env=env)
    assert out.returncode == 0, out.stdout[-2000:] + out.stderr[-4000:]
    assert expect in out.stdout
    assert "runtime error" not in out.stderr and "ERROR: AddressSanitizer" not in out.stderr, out.stderr[-4000:]
