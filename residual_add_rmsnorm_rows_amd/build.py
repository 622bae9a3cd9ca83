"""Build the HIP library ``librmsnorm_rows.so`` in-tree for gfx950.

Kernel translation units are compiled with hipcc (device code for gfx950
only); the host-only selector and C ABI are compiled with g++ against the HIP
runtime headers; everything is linked into one shared library next to this
file.  Compilation runs in parallel, one process per translation unit.  A small native driver,
``rn_decode_latency``, is linked against the library for decode timings.

Usage: ``python -m residual_add_rmsnorm_rows_amd.build`` (or ``build()``).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_NAME = "librmsnorm_rows.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
DECODE_LATENCY_PATH = os.path.join(PKG_DIR, "rn_decode_latency")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

# Packed fp32 VALU ops are kept out of generated code (-packed-fp32-ops);
# the host pass of hipcc warns that it does not know the feature, harmlessly.
# Each HIP translation unit gets a fixed compilation-unit ID (-cuid, below):
# by default clang derives it from the source file's absolute path, which
# would make the library's bytes depend on where the tree is checked out.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
HOST_FLAGS = [
    "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
    "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{INCLUDE}", f"-I{CSRC}",
]

ROW_VARIANTS = [  # (x dtype, out dtype, scale scheme, name)
    (x, out, qs, f"{xn}_{on}" + (f"_{qn}" if qn else ""))
    for x, xn in (("kBF16", "bf16"), ("kF32", "f32"))
    for out, on, qs, qn in (("kBF16", "bf16", "kQRow", ""), ("kF32", "f32", "kQRow", ""),
                            ("kFP8", "fp8", "kQRow", "row"), ("kFP8", "fp8", "kQGroup128", "g128"),
                            ("kFP8", "fp8", "kQMx32", "mx"), ("kFP4", "fp4", "kQMx32", "mx"),
                            ("kFP4", "fp4", "kQNv16", "nv"))
]


def _jobs():
    jobs = []
    for x, out, qs, name in ROW_VARIANTS:
        obj = os.path.join(BUILD_DIR, f"rows_{name}.o")
        cmd = [HIPCC, *HIP_FLAGS, f"-cuid=rows_{name}", f"-DRN_TU_X={x}", f"-DRN_TU_OUT={out}", f"-DRN_TU_QS={qs}",
               f"-DRN_TU_NAME={name}", "-c", os.path.join(CSRC, "rows_kernel.hip"), "-o", obj]
        jobs.append((obj, cmd))
    for name in ("heads_kernel", "act_kernel", "reference_kernels"):
        obj = os.path.join(BUILD_DIR, f"{name}.o")
        jobs.append((obj, [HIPCC, *HIP_FLAGS, f"-cuid={name}", "-c", os.path.join(CSRC, f"{name}.hip"), "-o", obj]))
    for src in ("select.cpp", "abi.cpp"):
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".o"))
        jobs.append((obj, ["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]))
    return jobs


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every translation unit and link the library; returns its path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    todo = _jobs()
    workers = jobs or min(len(todo), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda j: (j, _run(j[1])), todo))
    failed = [(j, out) for j, (rc, out) in results if rc != 0]
    for (obj, cmd), (rc, out) in results:
        if verbose or rc != 0:
            print(" ".join(cmd), file=sys.stderr)
            if out.strip():
                print(out, file=sys.stderr)
    if failed:
        raise RuntimeError(f"{len(failed)} translation unit(s) failed to compile: "
                           + ", ".join(os.path.basename(j[0]) for j, _ in failed))
    tmp = LIB_PATH + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
            *[obj for obj, _ in todo], f"-L{ROCM}/lib", "-lamdhip64"]
    rc, out = _run(link)
    if rc != 0:
        print(" ".join(link), file=sys.stderr)
        print(out, file=sys.stderr)
        raise RuntimeError("link failed")
    os.replace(tmp, LIB_PATH)
    # native decode-latency driver, linked against the library just built
    exe_tmp = DECODE_LATENCY_PATH + ".tmp"
    drv = ["g++", *HOST_FLAGS, os.path.join(CSRC, "decode_latency.cpp"), "-o", exe_tmp,
           f"-L{os.path.dirname(LIB_PATH)}", "-lrmsnorm_rows", "-Wl,-rpath,$ORIGIN", f"-L{ROCM}/lib", "-lamdhip64",
           f"-Wl,-rpath,{ROCM}/lib"]
    rc, out = _run(drv)
    if rc != 0:
        print(" ".join(drv), file=sys.stderr)
        print(out, file=sys.stderr)
        raise RuntimeError("decode-latency driver failed to build")
    os.replace(exe_tmp, DECODE_LATENCY_PATH)
    return LIB_PATH


def clean() -> None:
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv)
    print(path)
