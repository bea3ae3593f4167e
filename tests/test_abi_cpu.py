"""The C-ABI library loads, exports every function include/mla.h declares, and
rejects bad arguments on the host before anything is launched (no GPU needed).
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
LIB = os.path.join(ROOT, "mla_decode_paged_amd", "libmla.so")

MLA_OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        subprocess.run(["python", "-m", "mla_decode_paged_amd.build"], cwd=ROOT, check=True)
    import mla_decode_paged_amd as mla
    return mla.load()


def test_header_declares_the_path():
    names = declared_functions()
    for fn in ("mla_get_metadata", "mla_absorb_q", "mla_decode_paged", "mla_up_v", "mla_gather_pages", "mla_append_kv",
               "mla_last_error", "mla_num_slots", "mla_workspace_bytes", "mla_take_device_error"):
        assert fn in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (mla_\w+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing
    for f in declared_functions():
        getattr(lib, f)


def test_workspace_formula(lib):
    # fp16 partial rows [b + slots, M, 512], fp32 lse and fp32 row scales [b + slots, M],
    # each region padded to 256 bytes
    pad = lambda x: (x + 255) // 256 * 256
    for b, s_q, h, slots in [(128, 1, 128, 256), (3, 4, 128, 7), (5, 1, 16, 9)]:
        M = s_q * h
        assert lib.mla_workspace_bytes(b, s_q, h, slots) == pad((b + slots) * M * 512 * 2) + 2 * pad((b + slots) * M * 4)
    assert lib.mla_workspace_bytes(0, 1, 128, 8) == 0


FAKE = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: every case fails validation first


def _decode(lib, **kw):
    a = dict(q_lat=FAKE, q_lat_lo=None, q_pe=FAKE, kv=FAKE, num_pages=10, bt=FAKE, max_blocks=4, sl=FAKE, b=2,
             s_q=1, h=16, scale=0.07, causal=0, meta=FAKE, ns=FAKE, slots=8, ws=FAKE, ws_bytes=1 << 30, o=FAKE,
             lse=FAKE)
    a.update(kw)
    return lib.mla_decode_paged(a["q_lat"], a["q_lat_lo"], a["q_pe"], a["kv"], a["num_pages"], a["bt"],
                                a["max_blocks"], a["sl"], a["b"], a["s_q"], a["h"], a["scale"], a["causal"],
                                a["meta"], a["ns"], a["slots"], a["ws"], a["ws_bytes"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q_lat=None), INVALID, "NULL"),
    (dict(kv=None), INVALID, "NULL"),
    (dict(b=0), INVALID, "b must be"),
    (dict(s_q=9), INVALID, "s_q"),
    (dict(h=48), UNSUPPORTED, "h must be"),
    (dict(scale=0.0), INVALID, "softmax_scale"),
    (dict(scale=float("nan")), INVALID, "softmax_scale"),
    (dict(num_pages=0), INVALID, "num_pages"),
    (dict(slots=0), INVALID, "num_slots"),
    (dict(ws_bytes=1000), WORKSPACE, "workspace"),
    (dict(ws=ctypes.c_void_p((1 << 20) + 16)), INVALID, "aligned"),
    (dict(q_lat=ctypes.c_void_p((1 << 20) + 2)), INVALID, "aligned"),
])
def test_decode_rejects(lib, kw, code, msg):
    assert _decode(lib, **kw) == code
    assert msg in lib.mla_last_error().decode()


def test_other_calls_reject(lib):
    assert lib.mla_get_metadata(FAKE, 0, 8, 2, FAKE, FAKE, None) == INVALID
    assert lib.mla_get_metadata(FAKE, 9000, 8, 2, FAKE, FAKE, None) == INVALID
    assert lib.mla_get_metadata(FAKE, 4, 0, 2, FAKE, FAKE, None) == INVALID
    assert lib.mla_get_metadata(FAKE, 4, 8, -1, FAKE, FAKE, None) == INVALID
    assert lib.mla_get_metadata(None, 4, 8, 2, FAKE, FAKE, None) == INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, None, 2, 1, 100, None) == UNSUPPORTED
    assert lib.mla_absorb_q(None, FAKE, FAKE, None, 2, 1, 16, None) == INVALID
    assert lib.mla_absorb_q(FAKE, FAKE, FAKE, ctypes.c_void_p((1 << 20) + 8), 2, 1, 16, None) == INVALID
    assert lib.mla_up_v(FAKE, FAKE, None, 2, 1, 16, None) == INVALID
    assert lib.mla_up_v(FAKE, FAKE, FAKE, 2, 0, 16, None) == INVALID
    assert lib.mla_gather_pages(FAKE, 0, FAKE, 4, FAKE, 2, FAKE, FAKE, None) == INVALID
    assert lib.mla_gather_pages(FAKE, 4, FAKE, 4, FAKE, 2, None, FAKE, None) == INVALID
    assert lib.mla_append_kv(None, FAKE, 4, FAKE, 4, FAKE, 2, 1, None) == INVALID
    assert lib.mla_append_kv(FAKE, FAKE, 4, FAKE, 4, None, 2, 1, None) == INVALID
    assert lib.mla_append_kv(FAKE, FAKE, 4, FAKE, 4, FAKE, 0, 1, None) == INVALID
    assert lib.mla_append_kv(FAKE, FAKE, 4, FAKE, 4, FAKE, 2, 9, None) == INVALID
    assert lib.mla_append_kv(FAKE, FAKE, 0, FAKE, 4, FAKE, 2, 1, None) == INVALID
    assert lib.mla_append_kv(FAKE, FAKE, 4, FAKE, 0, FAKE, 2, 1, None) == INVALID
    assert lib.mla_append_kv(ctypes.c_void_p((1 << 20) + 8), FAKE, 4, FAKE, 4, FAKE, 2, 1, None) == INVALID
    assert lib.mla_num_slots(2, 1, 16, None) == INVALID
    assert lib.mla_take_device_error(None) == INVALID
    assert lib.mla_last_error().decode() != ""


def _absorb_plan(lib, **kw):
    a = dict(q_nope=FAKE, w_uk=FAKE, q_lat=FAKE, q_lo=None, b=2, s_q=1, h=16, sl=FAKE, slots=8, F=2, meta=FAKE,
             ns=FAKE)
    a.update(kw)
    return lib.mla_absorb_q_with_plan(a["q_nope"], a["w_uk"], a["q_lat"], a["q_lo"], a["b"], a["s_q"], a["h"],
                                      a["sl"], a["slots"], a["F"], a["meta"], a["ns"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q_nope=None), INVALID, "q_nope"),
    (dict(q_lo=ctypes.c_void_p((1 << 20) + 8)), INVALID, "aligned"),
    (dict(h=100), UNSUPPORTED, "h must be"),
    (dict(s_q=0), INVALID, "s_q"),
    (dict(sl=None), INVALID, "NULL"),
    (dict(meta=None), INVALID, "NULL"),
    (dict(b=9000), INVALID, "b must be"),
    (dict(slots=0), INVALID, "num_slots"),
    (dict(F=-1), INVALID, "split_overhead"),
])
def test_absorb_with_plan_rejects(lib, kw, code, msg):
    """The combined call applies the checks of both calls before anything is launched."""
    assert _absorb_plan(lib, **kw) == code
    assert msg in lib.mla_last_error().decode()


def _noalloc(lib, **kw):
    a = dict(q_lat=FAKE, q_lat_lo=None, q_pe=FAKE, kv=FAKE, num_pages=10, bt=FAKE, max_blocks=4, sl=FAKE, b=2,
             s_q=1, h=16, scale=0.07, causal=0, meta=FAKE, ns=FAKE, slots=8, o=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mla_decode_paged_noalloc(a["q_lat"], a["q_lat_lo"], a["q_pe"], a["kv"], a["num_pages"], a["bt"],
                                        a["max_blocks"], a["sl"], a["b"], a["s_q"], a["h"], a["scale"],
                                        a["causal"], a["meta"], a["ns"], a["slots"], a["o"], a["lse"], None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(q_lat=None), INVALID, "NULL"),
    (dict(lse=None), INVALID, "NULL"),
    (dict(h=48), UNSUPPORTED, "h must be"),
    (dict(scale=-1.0), INVALID, "softmax_scale"),
    (dict(o=ctypes.c_void_p((1 << 20) + 8)), INVALID, "aligned"),
    # 8192 sequences of 1024 rows: far more split partials than the built-in scratch holds
    (dict(b=8192, s_q=8, h=128, slots=256), WORKSPACE, "built-in scratch"),
])
def test_noalloc_rejects(lib, kw, code, msg):
    """The no-allocation decode entry applies the decode checks and refuses shapes whose split partials
    exceed its fixed scratch, before it touches the device."""
    assert _noalloc(lib, **kw) == code
    assert msg in lib.mla_last_error().decode()


def test_noalloc_scratch_size_matches_the_header(lib):
    import mla_decode_paged_amd as mla
    text = open(HEADER).read()
    m = re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == mla.NOALLOC_SCRATCH_BYTES
    # the largest default-slot workspaces of the benchmark workloads fit
    for b, s_q, h, slots in [(128, 1, 32, 256), (128, 1, 128, 256), (16, 1, 128, 256), (128, 2, 128, 128),
                             (32, 8, 128, 32)]:
        assert lib.mla_workspace_bytes(b, s_q, h, slots) <= mla.NOALLOC_SCRATCH_BYTES


def test_quantised_cache_calls_reject(lib):
    """The quantised-cache entry points check their arguments before anything is launched."""
    assert lib.mla_quantize_pages(None, 4, FAKE, None) == INVALID
    assert lib.mla_quantize_pages(FAKE, 0, FAKE, None) == INVALID
    assert lib.mla_quantize_pages(FAKE, 4, ctypes.c_void_p((1 << 20) + 8), None) == INVALID
    assert lib.mla_append_kv_fp8(FAKE, FAKE, 4, FAKE, 4, FAKE, 2, 9, None) == INVALID
    assert lib.mla_append_kv_fp8(FAKE, None, 4, FAKE, 4, FAKE, 2, 1, None) == INVALID
    assert lib.mla_append_kv_fp8(FAKE, ctypes.c_void_p((1 << 20) + 4), 4, FAKE, 4, FAKE, 2, 1, None) == INVALID
    args = [FAKE, None, FAKE, FAKE, 10, FAKE, 4, FAKE, 2, 1, 64, 0.07, 0, FAKE, FAKE, 8, FAKE, 1 << 30, FAKE, FAKE,
            None]
    assert lib.mla_decode_paged_fp8(*args) == UNSUPPORTED  # 64 rows: more than the 32 it is built for
    assert "at most 32 query rows" in lib.mla_last_error().decode()
    args[10] = 32
    args[16] = None
    assert lib.mla_decode_paged_fp8(*args) == INVALID      # no workspace
    args[16] = FAKE
    args[17] = 1000
    assert lib.mla_decode_paged_fp8(*args) == WORKSPACE


def test_quantised_page_constants():
    import mla_decode_paged_amd as mla
    text = open(HEADER).read()
    assert "#define MLA_FP8_ROW_BYTES 640" in text
    assert mla.FP8_ROW_BYTES == 640 and mla.FP8_PAGE_BYTES == 64 * 640 + 256 == 41216
    from oracle import kv_quant
    assert kv_quant.PAGE_BYTES == mla.FP8_PAGE_BYTES and kv_quant.ROW_BYTES == mla.FP8_ROW_BYTES
