"""Rules on the generated gfx950 code of every kernel translation unit.

CPU only: the device assembly comes from the build's own hipcc command lines
with ``-S --cuda-device-only`` in place of ``-c``, so it is the code the
library links.  Checked for every kernel:

- no instruction writes through the scalar data cache (scalar stores, scalar
  atomics, the cache's write-back or discard): every global write is a vector
  (buffer) store;
- no packed fp32 VALU instruction: the build turns that feature off, and this
  checks that the flag reaches every translation unit;
- no register spills to scratch memory: every kernel has an empty private
  segment and spills no VGPRs; SGPR spills, which land in VGPR lanes, are
  allowed only in the partial-input rows kernels (a buffer resource of 4
  SGPRs per slot next to the kernel arguments).
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from residual_add_rmsnorm_rows_amd import build as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.HIPCC), reason="hipcc not installed")

SCALAR_CACHE_WRITE = re.compile(
    r"^\s+(s_store\w*|s_buffer_store\w*|s_scratch_store\w*|s_atomic\w*|s_buffer_atomic\w*"
    r"|s_dcache_wb\w*|s_dcache_discard\w*)\b", re.M)
PACKED_F32 = re.compile(r"^\s+(v_pk_(?:add|mul|fma)_f32)\b", re.M)
KERNEL_NAME = re.compile(r"^\s+\.symbol:\s+(\S+)\.kd$", re.M)
META = {key: re.compile(rf"^\s+\.{key}:\s+(\d+)$", re.M)
        for key in ("private_segment_fixed_size", "sgpr_spill_count", "vgpr_spill_count")}


def _asm_job(job, out_dir):
    obj, cmd = job
    src = next((a for a in cmd if a.endswith(".hip")), None)
    if src is None:
        return None
    name = os.path.basename(obj)[:-2]
    cmd = [a for a in cmd if a not in ("-c", "-fPIC")]
    cut = cmd.index("-o")
    asm = os.path.join(out_dir, f"{name}.s")
    p = subprocess.run(cmd[:cut] + ["-S", "--cuda-device-only", "-o", asm],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    return name, p.returncode, p.stdout, asm


@pytest.fixture(scope="module")
def device_asm(tmp_path_factory):
    out_dir = str(tmp_path_factory.mktemp("isa"))
    with ThreadPoolExecutor(min(8, os.cpu_count() or 1)) as ex:
        results = [r for r in ex.map(lambda j: _asm_job(j, out_dir), B._jobs()) if r is not None]
    asm = {}
    for name, rc, log, path in results:
        assert rc == 0, f"{name}: hipcc failed\n{log[-2000:]}"
        with open(path) as f:
            asm[name] = f.read()
    yield asm
    shutil.rmtree(out_dir, ignore_errors=True)


def test_every_kernel_translation_unit_compiled(device_asm):
    hip_sources = {os.path.basename(o)[:-2] for o, c in B._jobs() if any(a.endswith(".hip") for a in c)}
    assert set(device_asm) == hip_sources
    for name, text in device_asm.items():
        assert KERNEL_NAME.search(text), f"{name}: no kernel metadata"


def test_no_write_through_the_scalar_data_cache(device_asm):
    bad = {name: sorted(set(SCALAR_CACHE_WRITE.findall(text))) for name, text in device_asm.items()}
    assert not {k: v for k, v in bad.items() if v}


def test_no_packed_fp32_instructions(device_asm):
    bad = {name: sorted(set(PACKED_F32.findall(text))) for name, text in device_asm.items()}
    assert not {k: v for k, v in bad.items() if v}


# rows_kernel<x, res, w, out, scheme, bias, NV, KP> with NV == 1 (these ask
# for 8 waves per SIMD) or KP in {2, 4, 8} (a buffer resource per slot): the
# compiler may move SGPRs past the budget into VGPR lanes (v_writelane /
# v_readlane, no memory); VGPR spills and scratch memory stay forbidden
# everywhere
SGPR_LANE_SPILL_OK = re.compile(r"rows_kernelI(?:Li\d+E){6}(?:Li1ELi\d+|Li\d+ELi[248])EEEvNS_7RowArgsE$")


def test_no_register_spills(device_asm):
    n_exempt = 0
    for name, text in device_asm.items():
        kernels = KERNEL_NAME.findall(text)
        n_exempt += sum(1 for k in kernels if SGPR_LANE_SPILL_OK.search(k))
        for key, pat in META.items():
            values = [int(v) for v in pat.findall(text)]
            assert len(values) == len(kernels), f"{name}: {key} missing for some kernel"
            bad = [k for k, v in zip(kernels, values)
                   if v and not (key == "sgpr_spill_count" and SGPR_LANE_SPILL_OK.search(k))]
            assert not bad, f"{name}: nonzero {key} in {bad}"
    assert n_exempt > 0  # the exemption names kernels that exist
