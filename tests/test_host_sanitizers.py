"""The host side of libmla under AddressSanitizer and UndefinedBehaviorSanitizer.

The library sources and tests/host_sanitize/abi_calls.cpp are compiled together
with the sanitizers on the host pass only (`-Xarch_host` before each
`-fsanitize=`; the device code is built as usual and never launched). The program
drives every entry point's argument checks, the error-message buffer (from
several threads) and the size queries over ordinary and extreme values; any
sanitizer report or failed check fails the test. No GPU is needed or used.
"""
import hashlib
import os
import shutil
import subprocess

import pytest

from mla_decode_paged_amd import build as mla_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HARNESS = os.path.join(ROOT, "tests", "host_sanitize", "abi_calls.cpp")
OUT_DIR = os.path.join(ROOT, "_build", "host_sanitize")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _sources():
    srcs = [os.path.join(mla_build.CSRC, s) for s in mla_build.SOURCES]
    headers = sorted(os.path.join(mla_build.CSRC, f) for f in os.listdir(mla_build.CSRC) if f.endswith(".h"))
    return srcs, headers + [os.path.join(ROOT, "include", "mla.h"), HARNESS]


def _build():
    cc = mla_build.hipcc()
    srcs, deps = _sources()
    h = hashlib.sha256()
    for f in srcs + deps:
        h.update(open(f, "rb").read())
    exe = os.path.join(OUT_DIR, f"abi_calls_{h.hexdigest()[:16]}")
    if os.path.exists(exe):
        return exe
    os.makedirs(OUT_DIR, exist_ok=True)
    procs, objs = [], []
    for src in srcs + [HARNESS]:
        obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
        flags = mla_build.COMMON + mla_build.PER_FILE.get(os.path.basename(src), []) if src != HARNESS else \
            ["-O1", "-std=c++17", "-fPIC"]
        cmd = [cc, *flags, *SAN, "-g", "-c", src, "-o", obj]
        if src == HARNESS:
            cmd.insert(1, "-x")
            cmd.insert(2, "hip")
            cmd.insert(3, f"--offload-arch={mla_build.ARCH}")
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    for src, p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, f"compiling {src} with sanitizers failed:\n{out[-4000:]}"
    for old in os.listdir(OUT_DIR):  # builds of earlier sources
        if old.startswith("abi_calls_") and not old.endswith(".o"):
            os.remove(os.path.join(OUT_DIR, old))
    tmp = exe + ".tmp"
    r = subprocess.run([cc, f"--offload-arch={mla_build.ARCH}", *SAN, *objs, "-o", tmp, "-lpthread"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    os.replace(tmp, exe)
    return exe


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the sanitized host code")
def test_host_entry_points_under_asan_and_ubsan():
    exe = _build()
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1:detect_stack_use_after_return=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["HIP_VISIBLE_DEVICES"] = ""  # host code only: the program never needs a device
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = r.stdout + r.stderr
    assert r.returncode == 0, report[-6000:]
    assert "host checks passed" in r.stdout
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "ERROR: LeakSanitizer"):
        assert marker not in report, report[-6000:]


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to build the sanitized host code")
@pytest.mark.parametrize("bug,marker", [
    ("int* p = new int[4]; int v = p[argc + 3]; delete[] p; return v;", "heap-buffer-overflow"),
    ("int x = 2147483647 - 1 + argc; return x + 1 > 0 ? 0 : 1;", "runtime error: signed integer overflow"),
])
def test_the_sanitizer_flags_catch_planted_host_bugs(tmp_path, bug, marker):
    """The same compiler flags on a planted host bug produce the report the test above looks for,
    so a clean run there means the checks were live."""
    src = tmp_path / "bug.cpp"
    src.write_text("#include <hip/hip_runtime.h>\nint main(int argc, char**) { " + bug + " }\n")
    exe = tmp_path / "bug"
    r = subprocess.run([mla_build.hipcc(), "-x", "hip", f"--offload-arch={mla_build.ARCH}", "-O1", *SAN, "-g",
                        str(src), "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=60)
    assert r.returncode != 0 and marker in r.stderr, r.stderr[-3000:]
