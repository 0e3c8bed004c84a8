"""Build the gfx950 HIP library ``libgdn.so`` in-tree with hipcc.

The library is one translation unit (``csrc/gdn_api.hip``) that includes every
kernel header; it is rebuilt from scratch on every call.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgdn.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed fp32 (v_pk_*_f32) code generation
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the kernels fit in 256 of them, and
    # accumulation registers would cost a copy for every tile that is reused
    # as an operand or rescaled
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-o", tmp, os.path.join(CSRC, "gdn_api.hip")]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (res.stdout + res.stderr).splitlines()
                     if "packed-fp32-ops' is not a recognized feature" not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
