"""Host-side checks of bench.py: its algorithmic byte counts (the roofline's
numerator) worked out by hand from each workload's tensors, and the command
line's refusals (no GPU needed)."""

import os
import subprocess
import sys

import bench
import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_workloads():
    # prefill 16384 x 8192: bf16 x in, f32 residual in and out, bf16 out, bf16 weight once
    assert bench.rownorm_bytes(WL.WORKLOADS["prefill_16384x8192"]) == 16384 * 8192 * (2 + 4 + 4 + 2) + 8192 * 2
    assert bench.rownorm_bytes(WL.WORKLOADS["prefill_16384x8192"]) == 1_610_629_120
    # fp8 prefill 8192 x 7168: bf16 x, bf16 residual in and out, fp8 codes, one float32 scale per row
    fp8 = WL.WORKLOADS["prefill_fp8_8192x7168"]
    assert bench.rownorm_bytes(fp8) == 8192 * (7168 * (2 + 2 + 2 + 1) + 4) + 7168 * 2 == 411_088_896
    # the block-scaled schemes on the same rows: per-128 float32, E8M0 per 32, fp4 codes + E4M3 per 16
    assert bench.rownorm_bytes(fp8, scale_scheme="group128") == 8192 * (7168 * 7 + 4 * 56) + 14336
    assert bench.rownorm_bytes(fp8, scale_scheme="mx32") == 8192 * (7168 * 7 + 224) + 14336
    from dataclasses import replace
    fp4 = replace(fp8, out_dtype="fp4_e2m1")
    assert bench.rownorm_bytes(fp4, scale_scheme="nv16") == 8192 * (7168 * 6.5 + 448) + 14336
    # QK-norm 4096 tokens x 32 heads x 128, in place: read and write every element, one weight
    assert bench.qknorm_bytes(WL.WORKLOADS["qknorm_4096x32x128"]) == 2 * 4096 * 32 * 128 * 2 + 128 * 2 == 67_109_120
    # 8 partials of 2048 x 8192 bf16, f32 residual in and out, bf16 out, bf16 weight
    p = WL.WORKLOADS["partials_8x2048x8192"]
    assert bench.partials_bytes(p) == 2048 * 8192 * (8 * 2 + 4 + 4 + 2) + 8192 * 2 == 436_224_000
    # the same with MXFP4 out: half a byte per code and one E8M0 byte per 32 elements
    assert bench.partials_bytes(replace(p, out_dtype="fp4_e2m1"), "mx32") == \
        2048 * (8192 * (8 * 2 + 4 + 4) + 8192 // 2 + 8192 // 32) + 8192 * 2


def _run(*args):
    env = dict(os.environ, WORLD_SIZE="1")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    out = _run("--gpus", "2")
    assert out.returncode == 2 and "one GPU only" in out.stderr


def test_bad_step_counts_are_refused():
    assert _run("--steps", "0").returncode == 2
    assert _run("--warmup", "-1").returncode == 2
