"""Register and scratch use of every kernel, from the compiler's resource report (CPU only).

Compiles each HIP source of the stage library for gfx950 with the build's flags and
-Rpass-analysis=kernel-resource-usage, and checks that no kernel uses scratch memory (register
spills go to per-lane scratch, which is slow and was once seen on a GEMM tile), and that the
attention kernels keep the occupancy their launch shapes assume.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from pipeline_stage_decoder_amd import build as B

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")

REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                    r"VGPRs Spill|SGPRs Spill): (\S+)")


def resource_report():
    """{kernel symbol: {field: value}} over every source of the library."""
    out = {}
    with tempfile.TemporaryDirectory() as tmp:
        procs = []
        for src in B.SOURCES:
            cmd = ["hipcc", *B.HIPFLAGS, "-c", os.path.join(B.CSRC, src), "-o", os.path.join(tmp, src + ".o"),
                   "-Rpass-analysis=kernel-resource-usage"]
            procs.append(subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT))
        for p in procs:
            text = p.communicate()[0].decode(errors="replace")
            assert p.returncode == 0, text[-2000:]
            name = None
            for m in REMARK.finditer(text):
                field, value = m.group(1), m.group(2)
                if field == "Function Name":
                    name = value
                    out[name] = {}
                elif name is not None:
                    out[name][field] = int(value)
    return out


@pytest.fixture(scope="module")
def report():
    return resource_report()


def test_no_kernel_spills_to_scratch(report):
    assert len(report) > 20
    spills = {k: v for k, v in report.items()
              if v.get("ScratchSize [bytes/lane]", 0) or v.get("VGPRs Spill", 0) or v.get("SGPRs Spill", 0)}
    assert not spills, spills


def test_bf16_and_f16_attention_keep_two_waves_per_simd(report):
    # the decode (plain and non-temporal loads), two-buffer prefill and 32-column prefill attention
    # kernels over 2-byte caches (KvFmt 0 = bf16, 2 = binary16) with head dim 128 must fit two
    # waves per SIMD (the three-buffer prefill runs only on grids of one work-group per CU)
    pat = r"k_attn_decodeILi128ELi[02]ELb[01]E|k_attn_prefillILi128ELi[02]ELi2E|k_attn_prefill32ILi128ELi[02]E"
    seen = 0
    for k, v in report.items():
        if re.search(pat, k):
            seen += 1
            assert v["Occupancy [waves/SIMD]"] >= 2, (k, v)
    assert seen == 8
