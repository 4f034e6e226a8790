"""Compile-time resource checks of the decode kernel variants (no GPU needed).

hipcc's resource-usage remarks for gfx950, taken with the library's own flags:
- no decode-kernel variant uses scratch memory (register spills);
- every single-row vector-path variant (one query row per KV head: the MHA and
  fp8 workloads) keeps at least four waves per SIMD, i.e. two 8-wave workgroups
  per CU.

The split plan sizes the grid from the occupancy the runtime reports, so a
variant that drops below that gets half the splits; a source change that
raised the fp8 KIVI variant from 112 to 136 VGPRs cost its step 19%.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from gqa_decode_attention_paged_amd import build

NAME = re.compile(r"paged_decode_kernelILi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)E")


@pytest.fixture(scope="module")
def resources():
    try:
        hipcc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [hipcc, *flags, "--offload-device-only", "-c",
               "-Rpass-analysis=kernel-resource-usage", build.DECODE_SOURCE,
               "-o", os.path.join(tmp, "k.o")]
        res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    kernels, cur = {}, None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"(VGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            kernels[cur][m.group(1).split()[0]] = int(m.group(2))
    decode = {}
    for name, r in kernels.items():
        m = NAME.search(name)
        if m:
            decode[tuple(int(x) for x in m.groups())] = r     # (D, BS, M, KV, WAVES)
    assert len(decode) >= 100, f"found {len(decode)} decode variants"
    return decode


def test_no_decode_variant_spills(resources):
    spills = {k: r for k, r in resources.items() if r.get("ScratchSize", 0) != 0}
    assert not spills, f"variants with scratch (D, BS, M, KV, WAVES): {spills}"


def test_single_row_vector_variants_keep_four_waves_per_simd(resources):
    rows1 = {k: r for k, r in resources.items() if k[2] == 1}
    assert len(rows1) >= 20
    low = {k: r for k, r in rows1.items() if r["Occupancy"] < 4}
    assert not low, f"single-row variants below 4 waves/SIMD (D, BS, M, KV, WAVES): {low}"
