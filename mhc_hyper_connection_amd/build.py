"""Builds libmhc.so (the C-ABI library) in-tree with hipcc for gfx950.

    python -m mhc_hyper_connection_amd.build

Every HIP translation unit is compiled with the packed-fp32 instructions disabled
(the compiler otherwise forms v_pk_* fp32 operations from plain float code) and with
matrix-core operands in VGPRs (see HIP_FLAGS).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libmhc.so")
ARCH = os.environ.get("MHC_OFFLOAD_ARCH", "gfx950")

SOURCES = [os.path.join(CSRC, "mhc_kernels.hip"), os.path.join(CSRC, "mhc_bwd.hip"), os.path.join(CSRC, "mhc_post.hip"),
           os.path.join(CSRC, "mhc_scratch.hip"), os.path.join(CSRC, "mhc_api.cpp")]
# -amdgpu-mfma-vgpr-form=1 keeps matrix-core sources and accumulators in ordinary VGPRs.
# With the default accumulation-register form, this toolchain's code for the projection
# kernel produced wrong sums on gfx950 (deterministically, for every schedule tried); the
# VGPR form is correct and the GPU parity tests guard it.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-mllvm", "-amdgpu-mfma-vgpr-form=1",
             "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmhc.so")


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles). Returns the path of libmhc.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-o", tmp, *SOURCES]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
