"""Every kernel of the library compiles for gfx950 without register spills.

A spill is a scratch store and reload; the reload's wait (vmcnt) also waits
for every global load the wave has in flight, which in the scan's pipelined
waves (loads issued one to three chunks ahead) turns prefetching into
waiting.  The check compiles the library's one translation unit with the
build's own flags and reads hipcc's per-kernel resource remarks.  CPU only
(hipcc cross-compiles); skipped where hipcc is absent.
"""
import os
import re
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

from gated_delta_rule_16_amd import build as gbuild  # noqa: E402


def _remarks(tmp_path):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    flags = [f for f in gbuild.HIPCC_FLAGS if f != "-shared"]
    cmd = [hipcc, *flags, "--cuda-device-only", "-c", "-Rpass-analysis=kernel-resource-usage",
           "-o", str(tmp_path / "gdn_api.o"), os.path.join(gbuild.CSRC, "gdn_api.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-2000:]
    return res.stderr


def test_no_kernel_spills(tmp_path):
    out = _remarks(tmp_path)
    names = re.findall(r"remark: Function Name: (\S+)", out)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", out)]
    vspill = [int(x) for x in re.findall(r"VGPRs Spill: (\d+)", out)]
    assert names and len(names) == len(scratch) == len(vspill), (len(names), len(scratch), len(vspill))
    bad = [(n, s, v) for n, s, v in zip(names, scratch, vspill) if s or v]
    assert not bad, bad
