"""Build libmla.so (the HIP kernels and the C ABI of include/mla.h) for gfx950.

    python -m mla_decode_paged_amd.build

Compiles every source under csrc/ with hipcc into the package directory, so the
library travels with the source tree. Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
ARCH = "gfx950"

SOURCES = ["mla_decode.hip", "mla_metadata.hip", "mla_gemm.hip"]
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions stay off: hipcc would otherwise form them from float code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]
# The decode kernel keeps its 256 output accumulators in AGPRs through inline
# asm; every other MFMA in that file must then use the VGPR form so that the
# score tile and the query fragments stay in VGPRs.
# The decode kernel also keeps every branch wave-uniform (see its divergence
# note); the atomic optimizer would turn each uniform atomic into a one-lane
# region, so it is off there.
PER_FILE = {"mla_decode.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form",
                               "-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmla)")


def build(verbose: bool = True) -> str:
    cc = hipcc()
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmp:
        objs = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            cmd = [cc, *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print("[mla build]", " ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                sys.stderr.write(r.stdout + r.stderr)
                raise RuntimeError(f"hipcc failed on {src}")
            objs.append(obj)
        tmp_lib = os.path.join(tmp, "libmla.so")
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        if verbose:
            print("[mla build]", " ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc link failed")
        shutil.copyfile(tmp_lib, LIB + ".tmp")
        os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
