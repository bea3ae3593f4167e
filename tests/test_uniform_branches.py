"""The attention kernels keep every branch uniform over the wave.

The row-block decode kernel once faulted the GPU from inside a lane-masked
region: under full register pressure the compiler had parked a live value
around a per-lane branch and reloaded it inside that region, so only the active
lanes got it back. Since then the decode, token-split and combine kernels have
no per-lane branch at all (padding rows repeat a valid row, stores past the
valid rows are dropped by buffer bounds, selects replace ifs, counts that decide
a branch are scalar loads). This test compiles mla_decode.hip for gfx950 with
the library's own flags to assembly, on the CPU, and checks that those kernels
contain no instruction that opens a lane-masked region (the s_*_saveexec
family). The small append kernel, which does branch per lane, shows that the
check sees such regions. No GPU is needed.
"""
import hashlib
import os
import re
import subprocess

import pytest

from mla_decode_paged_amd import build as mla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "isa")
UNIFORM = re.compile(r"mla_decode_kernel|mla_decode_tsplit_kernel|mla_combine_kernel")
MASKED = re.compile(r"\bs_(and|or|xor|andn2|orn2|nand|nor|xnor|andn1|orn1)_saveexec_b(32|64)\b")


def _assembly():
    src = os.path.join(mla_build.CSRC, "mla_decode.hip")
    h = hashlib.sha256()
    for f in sorted(os.listdir(mla_build.CSRC)):
        if f == "mla_decode.hip" or f.endswith(".h"):
            h.update(open(os.path.join(mla_build.CSRC, f), "rb").read())
    h.update(open(os.path.join(ROOT, "include", "mla.h"), "rb").read())
    h.update(" ".join(mla_build.COMMON + mla_build.PER_FILE.get("mla_decode.hip", [])).encode())
    out = os.path.join(OUT_DIR, f"mla_decode_{h.hexdigest()[:16]}.s")
    if not os.path.exists(out):
        os.makedirs(OUT_DIR, exist_ok=True)
        for old in os.listdir(OUT_DIR):  # assembly of earlier sources
            os.remove(os.path.join(OUT_DIR, old))
        cmd = [mla_build.hipcc(), *mla_build.COMMON, *mla_build.PER_FILE.get("mla_decode.hip", []),
               "--cuda-device-only", "-S", src, "-o", out + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"compiling mla_decode.hip to assembly failed:\n{r.stderr[-4000:]}"
        os.replace(out + ".tmp", out)
    return open(out).read()


def _functions(asm: str) -> dict:
    """Kernel symbol -> its instruction lines."""
    funcs, cur = {}, None
    for line in asm.split("\n"):
        m = re.match(r"^(_Z\S+):", line)
        if m:
            cur = m.group(1)
            funcs[cur] = []
            continue
        if line.startswith(".Lfunc_end"):
            cur = None
        elif cur is not None:
            funcs[cur].append(line.strip())
    return funcs


@pytest.fixture(scope="module")
def kernels():
    return _functions(_assembly())


def test_attention_kernels_open_no_lane_masked_region(kernels):
    names = [k for k in kernels if UNIFORM.search(k)]
    # the row-block kernel (two widths), the token-split kernel (two cache formats), the combine (two layouts)
    assert len(names) == 6, names
    bad = {k: [l for l in kernels[k] if MASKED.search(l)] for k in names}
    bad = {k: v for k, v in bad.items() if v}
    assert not bad, f"lane-masked regions in {sorted(bad)}: {[v[:3] for v in bad.values()]}"


def test_the_check_sees_lane_masked_regions(kernels):
    append = [k for k in kernels if "mla_append_kernel" in k]
    assert append and any(MASKED.search(l) for l in kernels[append[0]])
