"""Compile-time resource checks of the HIP kernels (CPU only: hipcc cross-compiles gfx950).

The split kernels keep several 32-token sub-tiles of loads in flight per wave
and wait for each with a partial vector-memory count; a register spill to
scratch memory would add scratch loads to that count and serialise the
pipeline. Every kernel must therefore compile without vector-register spills
and without scratch memory, and the loader/compute kernel must fit two waves
per SIMD (at most 256 VGPRs). Scalar registers may spill only in the split
kernel's in-kernel-merge instances, and only into lanes of vector registers
(no scratch): their merge epilogue runs once per workgroup after the
streaming loops, and the spill code sits at kernel entry and in that epilogue.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from latent_kv_cache_amd import build

pytestmark = pytest.mark.skipif(shutil.which(build.hipcc()) is None and not os.path.exists(build.hipcc()),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def remarks():
    text = ""
    with tempfile.TemporaryDirectory() as tmp:
        for src in build.HIP_SOURCES:
            cmd = [build.hipcc(), *build.HIP_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
                   os.path.join(build.CSRC, src), "-o", os.path.join(tmp, src + ".o")]
            res = subprocess.run(cmd, capture_output=True, text=True)
            assert res.returncode == 0, res.stderr[-2000:]
            text += res.stdout + res.stderr
    kernels = {}
    name = None
    for line in text.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            kernels[name] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|VGPRs Spill|SGPRs Spill|ScratchSize \[bytes/lane\]|"
                      r"Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            kernels[name][m.group(1)] = int(m.group(2))
    return kernels


def test_every_kernel_is_reported(remarks):
    names = " ".join(remarks)
    for kern in ("mlra_split_pc", "mlra_split_valu", "mlra_combine",
                 "mlra_append", "mlra_outproj_pack", "mlra_outproj", "mlra_outproj_reduce",
                 "mlra_prefill", "mlra_prefill_merge"):
        assert kern in names


def _in_kernel_merge(name):
    # mlra_split_pc<..., bool FUSED = true>: the mangled name ends its
    # template arguments with Lb1E
    return "mlra_split_pc" in name and "Lb1EE" in name


def test_no_kernel_spills(remarks):
    spilled = {k: v for k, v in remarks.items()
               if v.get("VGPRs Spill", 0) or v.get("ScratchSize [bytes/lane]", 0)
               or (v.get("SGPRs Spill", 0) and not _in_kernel_merge(k))}
    assert not spilled, spilled
    assert any(_in_kernel_merge(k) for k in remarks)


def test_loader_compute_kernel_runs_two_waves_per_simd(remarks):
    pc = {k: v for k, v in remarks.items() if "mlra_split_pc" in k}
    assert pc
    for k, v in pc.items():
        assert v["VGPRs"] + v.get("AGPRs", 0) <= 256, (k, v)


def test_prefill_kernel_runs_two_waves_per_simd(remarks):
    pf = {k: v for k, v in remarks.items() if "mlra_prefill" in k and "merge" not in k}
    assert len(pf) == 4  # latent 64/128 x RoPE 32/64
    for k, v in pf.items():
        assert v["VGPRs"] + v.get("AGPRs", 0) <= 256, (k, v)
