"""Python binding of libmla (include/mla.h): paged MLA decode on MI355X.

Argument marshalling only. Every step runs in the HIP kernels of libmla.so;
PyTorch supplies device memory and the current stream. Nothing here computes
on the CPU, and every call raises if the library is missing or returns an
error.

One decode step of one layer:

    tile_meta, num_splits = get_metadata(cache_seqlens)          # once per step
    q_lat, q_lat_lo = absorb_q(q_nope, w_uk)
    o_lat, lse = decode_paged(q_lat, q_pe, kv_cache, block_table, cache_seqlens,
                              tile_meta, num_splits, softmax_scale, causal,
                              q_lat_lo=q_lat_lo)
    o = up_v(o_lat, w_uv)

bf16 tensors are torch.bfloat16 (int16/uint16 views are accepted too).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["load", "last_error", "num_slots", "workspace_bytes", "get_metadata", "absorb_q", "absorb_q_with_plan",
           "decode_paged", "decode_paged_noalloc", "NOALLOC_SCRATCH_BYTES", "quantize_pages", "append_kv_fp8",
           "decode_paged_fp8", "FP8_ROW_BYTES", "FP8_PAGE_BYTES",
           "up_v", "gather_pages", "append_kv", "take_device_error", "MLAError", "LIB_PATH", "SPLIT_OVERHEAD",
           "SPLIT_OVERHEAD_FEW_ROWS", "SPLIT_OVERHEAD_ROW_BLOCKS", "default_split_overhead",
           "PAGE_TOKENS", "D_LATENT", "D_ROPE", "D_ROW", "D_NOPE", "MLA_DEVERR_PAGE_ID",
           "MLA_DEVERR_SEQ_TOO_LONG", "MLA_DEVERR_SHORT_SEQ"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
PAGE_TOKENS, D_LATENT, D_ROPE, D_ROW, D_NOPE = 64, 512, 64, 576, 128
# device error bits (MLA_DEVERR_* of include/mla.h)
MLA_DEVERR_PAGE_ID, MLA_DEVERR_SEQ_TOO_LONG, MLA_DEVERR_SHORT_SEQ = 1, 2, 4
META_WORDS = 8
# quantised cache page (MLA_FP8_* of include/mla.h): 64 rows of 640 bytes, then 64 fp32 scales
FP8_ROW_BYTES = 640
FP8_PAGE_BYTES = 64 * FP8_ROW_BYTES + 64 * 4
# MLA_NOALLOC_SCRATCH_BYTES of include/mla.h: the built-in scratch of decode_paged_noalloc
NOALLOC_SCRATCH_BYTES = 72 << 20
# Fixed cost of one sequence piece in the split plan, in pages: a piece's
# query loads, first-tile latency, epilogue stores and share of the merge,
# measured on MI355X against the per-page cost of the kernel that runs it.
# Row blocks of 128 rows (a sweep of 0..8 on the 128-head workload is
# fastest at 5-6):
SPLIT_OVERHEAD = 6
# At most 32 rows (the token-split kernel, whose pages cost about half as
# much and whose pieces start in a shared burst of first-tile loads; a sweep
# of 0..16 on the 32-head workload spans 30.1-33.1 us, 30.7 at 2):
SPLIT_OVERHEAD_FEW_ROWS = 2
# More than 128 rows (several row blocks per slot, speculative verify with
# 8 query tokens at 128 heads: F = 2/4/6/10/16 give 202.8/195.0/200.7/213.0/
# 231.4 us per call; 2 causal tokens with equal lengths do not split):
SPLIT_OVERHEAD_ROW_BLOCKS = 4

_lib = None
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class MLAError(RuntimeError):
    pass


def load():
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MLAError(f"{LIB_PATH} is missing: build it with `python -m mla_decode_paged_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "mla_last_error": (ctypes.c_char_p, []),
        "mla_num_slots": (_I, [_I, _I, _I, ctypes.POINTER(_I)]),
        "mla_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
        "mla_get_metadata": (_I, [_P, _I, _I, _I, _P, _P, _P]),
        "mla_absorb_q": (_I, [_P, _P, _P, _P, _I, _I, _I, _P]),
        "mla_absorb_q_with_plan": (_I, [_P, _P, _P, _P, _I, _I, _I, _P, _I, _I, _P, _P, _P]),
        "mla_decode_paged": (_I, [_P, _P, _P, _P, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _I, _P, _SZ,
                                  _P, _P, _P]),
        "mla_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _I,
                                          _P, _P, _P]),
        "mla_decode_paged_fp8": (_I, [_P, _P, _P, _P, _I64, _P, _I, _P, _I, _I, _I, _F, _I, _P, _P, _I, _P, _SZ,
                                      _P, _P, _P]),
        "mla_quantize_pages": (_I, [_P, _I64, _P, _P]),
        "mla_append_kv_fp8": (_I, [_P, _P, _I64, _P, _I, _P, _I, _I, _P]),
        "mla_up_v": (_I, [_P, _P, _P, _I, _I, _I, _P]),
        "mla_gather_pages": (_I, [_P, _I64, _P, _I, _P, _I, _P, _P, _P]),
        "mla_append_kv": (_I, [_P, _P, _I64, _P, _I, _P, _I, _I, _P]),
        "mla_take_device_error": (_I, [ctypes.POINTER(_I)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def last_error() -> str:
    return load().mla_last_error().decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise MLAError(f"{what} failed ({rc}): {last_error()}")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: torch.Tensor | None, name: str, dtypes=None, shape=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise MLAError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MLAError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise MLAError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MLAError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return ctypes.c_void_p(t.data_ptr())


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_I32 = (torch.int32,)


def num_slots(b: int, s_q: int, h: int) -> int:
    out = _I(0)
    _check(load().mla_num_slots(b, s_q, h, ctypes.byref(out)), "mla_num_slots")
    return out.value


def workspace_bytes(b: int, s_q: int, h: int, slots: int) -> int:
    n = load().mla_workspace_bytes(b, s_q, h, slots)
    if n == 0:
        raise MLAError("mla_workspace_bytes: bad arguments")
    return n


def default_split_overhead(s_q: int, h: int) -> int:
    m = s_q * h
    if m <= 32:
        return SPLIT_OVERHEAD_FEW_ROWS
    return SPLIT_OVERHEAD if m <= 128 else SPLIT_OVERHEAD_ROW_BLOCKS


def get_metadata(cache_seqlens: torch.Tensor, slots: int | None = None, s_q: int = 1, h: int = 128,
                 split_overhead: int | None = None, out=None):
    """Split-KV plan: (tile_meta int32 [slots, 8], num_splits int32 [b + 1])."""
    b = cache_seqlens.numel()
    if split_overhead is None:
        split_overhead = default_split_overhead(s_q, h)
    if slots is None:
        slots = num_slots(b, s_q, h) if out is None else out[0].shape[0]
    dev = cache_seqlens.device
    if out is None:
        tile_meta = torch.empty((slots, META_WORDS), dtype=torch.int32, device=dev)
        num_splits = torch.empty((b + 1,), dtype=torch.int32, device=dev)
    else:
        tile_meta, num_splits = out
    _check(load().mla_get_metadata(_ptr(cache_seqlens, "cache_seqlens", _I32), b, slots, split_overhead,
                                   _ptr(tile_meta, "tile_meta", _I32, (slots, META_WORDS)),
                                   _ptr(num_splits, "num_splits", _I32, (b + 1,)), _stream()),
           "mla_get_metadata")
    return tile_meta, num_splits


def absorb_q(q_nope: torch.Tensor, w_uk: torch.Tensor, lo: bool = True, out=None):
    """q_lat = q_nope @ W_UK per head, bf16 (and its bf16 rounding residue if lo)."""
    b, s_q, h, dn = q_nope.shape
    dev = q_nope.device
    if out is None:
        q_lat = torch.empty((b, s_q, h, D_LATENT), dtype=torch.bfloat16, device=dev)
        q_lo = torch.empty_like(q_lat) if lo else None
    else:
        q_lat, q_lo = out
    _check(load().mla_absorb_q(_ptr(q_nope, "q_nope", _BF16, (b, s_q, h, D_NOPE)),
                               _ptr(w_uk, "w_uk", _BF16, (h, D_NOPE, D_LATENT)),
                               _ptr(q_lat, "q_lat", _BF16, (b, s_q, h, D_LATENT)),
                               _ptr(q_lo, "q_lat_lo", _BF16, (b, s_q, h, D_LATENT)), b, s_q, h, _stream()),
           "mla_absorb_q")
    return q_lat, q_lo


def absorb_q_with_plan(q_nope: torch.Tensor, w_uk: torch.Tensor, cache_seqlens: torch.Tensor,
                       slots: int | None = None, split_overhead: int | None = None, lo: bool = True, out=None):
    """get_metadata and absorb_q in one launch (the first layer of a step):
    ((q_lat, q_lat_lo), (tile_meta, num_splits)). ``out`` is ((q_lat, q_lo), (tile_meta, num_splits))."""
    b, s_q, h, dn = q_nope.shape
    dev = q_nope.device
    if cache_seqlens.numel() != b:
        raise MLAError(f"cache_seqlens has {cache_seqlens.numel()} entries, expected {b}")
    if split_overhead is None:
        split_overhead = default_split_overhead(s_q, h)
    if out is None:
        if slots is None:
            slots = num_slots(b, s_q, h)
        q_lat = torch.empty((b, s_q, h, D_LATENT), dtype=torch.bfloat16, device=dev)
        q_lo = torch.empty_like(q_lat) if lo else None
        tile_meta = torch.empty((slots, META_WORDS), dtype=torch.int32, device=dev)
        num_splits = torch.empty((b + 1,), dtype=torch.int32, device=dev)
    else:
        (q_lat, q_lo), (tile_meta, num_splits) = out
        slots = tile_meta.shape[0]
    _check(load().mla_absorb_q_with_plan(_ptr(q_nope, "q_nope", _BF16, (b, s_q, h, D_NOPE)),
                                         _ptr(w_uk, "w_uk", _BF16, (h, D_NOPE, D_LATENT)),
                                         _ptr(q_lat, "q_lat", _BF16, (b, s_q, h, D_LATENT)),
                                         _ptr(q_lo, "q_lat_lo", _BF16, (b, s_q, h, D_LATENT)), b, s_q, h,
                                         _ptr(cache_seqlens, "cache_seqlens", _I32), slots, split_overhead,
                                         _ptr(tile_meta, "tile_meta", _I32, (slots, META_WORDS)),
                                         _ptr(num_splits, "num_splits", _I32, (b + 1,)), _stream()),
           "mla_absorb_q_with_plan")
    return (q_lat, q_lo), (tile_meta, num_splits)


def decode_paged(q_lat, q_pe, kv_cache, block_table, cache_seqlens, tile_meta, num_splits, softmax_scale,
                 causal, q_lat_lo=None, workspace=None, out=None):
    """Paged absorbed-form decode: (o_lat bf16 [b, s_q, h, 512], lse fp32 [b, s_q, h])."""
    if q_lat.dim() != 4 or tile_meta.dim() != 2:
        raise MLAError(f"q_lat must be [b, s_q, h, {D_LATENT}] and tile_meta [slots, {META_WORDS}]")
    b, s_q, h, _ = q_lat.shape
    slots = tile_meta.shape[0]
    dev = q_lat.device
    need = workspace_bytes(b, s_q, h, slots)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    if out is None:
        o_lat = torch.empty((b, s_q, h, D_LATENT), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((b, s_q, h), dtype=torch.float32, device=dev)
    else:
        o_lat, lse = out
    if kv_cache.dim() != 3 or tuple(kv_cache.shape[1:]) != (PAGE_TOKENS, D_ROW):
        raise MLAError(f"kv_cache must be [num_pages, {PAGE_TOKENS}, {D_ROW}]")
    if block_table.dim() != 2:
        raise MLAError(f"block_table must be [b, max_blocks], got shape {tuple(block_table.shape)}")
    _check(load().mla_decode_paged(
        _ptr(q_lat, "q_lat", _BF16, (b, s_q, h, D_LATENT)), _ptr(q_lat_lo, "q_lat_lo", _BF16, (b, s_q, h, D_LATENT)),
        _ptr(q_pe, "q_pe", _BF16, (b, s_q, h, D_ROPE)), _ptr(kv_cache, "kv_cache", _BF16), kv_cache.shape[0],
        _ptr(block_table, "block_table", _I32, (b, block_table.shape[1])), block_table.shape[1],
        _ptr(cache_seqlens, "cache_seqlens", _I32, (b,)), b, s_q, h, float(softmax_scale), int(bool(causal)),
        _ptr(tile_meta, "tile_meta", _I32, (slots, META_WORDS)), _ptr(num_splits, "num_splits", _I32, (b + 1,)),
        slots,
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(o_lat, "o_lat", _BF16, (b, s_q, h, D_LATENT)), _ptr(lse, "lse", (torch.float32,), (b, s_q, h)),
        _stream()), "mla_decode_paged")
    return o_lat, lse


def decode_paged_noalloc(q_lat, q_pe, kv_cache, block_table, cache_seqlens, tile_meta, num_splits, softmax_scale,
                         causal, q_lat_lo=None, out=None):
    """decode_paged without a workspace: the split partials use the library's fixed per-GPU scratch
    (mla_decode_paged_noalloc). Pass ``out`` to allocate nothing at all."""
    if q_lat.dim() != 4 or tile_meta.dim() != 2 or block_table.dim() != 2:
        raise MLAError(f"q_lat must be [b, s_q, h, {D_LATENT}], tile_meta [slots, {META_WORDS}] and "
                       "block_table [b, max_blocks]")
    b, s_q, h, _ = q_lat.shape
    slots = tile_meta.shape[0]
    dev = q_lat.device
    if out is None:
        o_lat = torch.empty((b, s_q, h, D_LATENT), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((b, s_q, h), dtype=torch.float32, device=dev)
    else:
        o_lat, lse = out
    if kv_cache.dim() != 3 or tuple(kv_cache.shape[1:]) != (PAGE_TOKENS, D_ROW):
        raise MLAError(f"kv_cache must be [num_pages, {PAGE_TOKENS}, {D_ROW}]")
    _check(load().mla_decode_paged_noalloc(
        _ptr(q_lat, "q_lat", _BF16, (b, s_q, h, D_LATENT)), _ptr(q_lat_lo, "q_lat_lo", _BF16, (b, s_q, h, D_LATENT)),
        _ptr(q_pe, "q_pe", _BF16, (b, s_q, h, D_ROPE)), _ptr(kv_cache, "kv_cache", _BF16), kv_cache.shape[0],
        _ptr(block_table, "block_table", _I32, (b, block_table.shape[1])), block_table.shape[1],
        _ptr(cache_seqlens, "cache_seqlens", _I32, (b,)), b, s_q, h, float(softmax_scale), int(bool(causal)),
        _ptr(tile_meta, "tile_meta", _I32, (slots, META_WORDS)), _ptr(num_splits, "num_splits", _I32, (b + 1,)),
        slots, _ptr(o_lat, "o_lat", _BF16, (b, s_q, h, D_LATENT)),
        _ptr(lse, "lse", (torch.float32,), (b, s_q, h)), _stream()), "mla_decode_paged_noalloc")
    return o_lat, lse


def quantize_pages(kv_cache, out=None):
    """bf16 paged cache [num_pages, 64, 576] -> the quantised page format, uint8 [num_pages, FP8_PAGE_BYTES]."""
    if kv_cache.dim() != 3 or tuple(kv_cache.shape[1:]) != (PAGE_TOKENS, D_ROW):
        raise MLAError(f"kv_cache must be [num_pages, {PAGE_TOKENS}, {D_ROW}]")
    n = kv_cache.shape[0]
    kv8 = out if out is not None else torch.empty((n, FP8_PAGE_BYTES), dtype=torch.uint8, device=kv_cache.device)
    _check(load().mla_quantize_pages(_ptr(kv_cache, "kv_cache", _BF16), n,
                                     _ptr(kv8, "kv_fp8", (torch.uint8,), (n, FP8_PAGE_BYTES)), _stream()),
           "mla_quantize_pages")
    return kv8


def append_kv_fp8(new_rows, kv_fp8, block_table, cache_seqlens):
    """append_kv into a quantised cache uint8 [num_pages, FP8_PAGE_BYTES] (each new row quantised)."""
    if new_rows.dim() != 3 or new_rows.shape[2] != D_ROW:
        raise MLAError(f"new_rows has shape {tuple(new_rows.shape)}, expected [b, s_q, {D_ROW}]")
    if kv_fp8.dim() != 2 or kv_fp8.shape[1] != FP8_PAGE_BYTES or block_table.dim() != 2:
        raise MLAError(f"kv_fp8 must be [num_pages, {FP8_PAGE_BYTES}] and block_table [b, max_blocks]")
    b, s_q = new_rows.shape[0], new_rows.shape[1]
    _check(load().mla_append_kv_fp8(_ptr(new_rows, "new_rows", _BF16), _ptr(kv_fp8, "kv_fp8", (torch.uint8,)),
                                    kv_fp8.shape[0], _ptr(block_table, "block_table", _I32, (b, block_table.shape[1])),
                                    block_table.shape[1], _ptr(cache_seqlens, "cache_seqlens", _I32, (b,)), b, s_q,
                                    _stream()), "mla_append_kv_fp8")
    return kv_fp8


def decode_paged_fp8(q_lat, q_pe, kv_fp8, block_table, cache_seqlens, tile_meta, num_splits, softmax_scale,
                     causal, q_lat_lo=None, workspace=None, out=None):
    """decode_paged over a quantised cache uint8 [num_pages, FP8_PAGE_BYTES] (at most 32 query rows per
    sequence): (o_lat bf16 [b, s_q, h, 512], lse fp32 [b, s_q, h])."""
    if q_lat.dim() != 4 or tile_meta.dim() != 2 or block_table.dim() != 2:
        raise MLAError(f"q_lat must be [b, s_q, h, {D_LATENT}], tile_meta [slots, {META_WORDS}] and "
                       "block_table [b, max_blocks]")
    if kv_fp8.dim() != 2 or kv_fp8.shape[1] != FP8_PAGE_BYTES:
        raise MLAError(f"kv_fp8 must be [num_pages, {FP8_PAGE_BYTES}]")
    b, s_q, h, _ = q_lat.shape
    slots = tile_meta.shape[0]
    dev = q_lat.device
    need = workspace_bytes(b, s_q, h, slots)
    if workspace is None:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    if out is None:
        o_lat = torch.empty((b, s_q, h, D_LATENT), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((b, s_q, h), dtype=torch.float32, device=dev)
    else:
        o_lat, lse = out
    _check(load().mla_decode_paged_fp8(
        _ptr(q_lat, "q_lat", _BF16, (b, s_q, h, D_LATENT)), _ptr(q_lat_lo, "q_lat_lo", _BF16, (b, s_q, h, D_LATENT)),
        _ptr(q_pe, "q_pe", _BF16, (b, s_q, h, D_ROPE)), _ptr(kv_fp8, "kv_fp8", (torch.uint8,)), kv_fp8.shape[0],
        _ptr(block_table, "block_table", _I32, (b, block_table.shape[1])), block_table.shape[1],
        _ptr(cache_seqlens, "cache_seqlens", _I32, (b,)), b, s_q, h, float(softmax_scale), int(bool(causal)),
        _ptr(tile_meta, "tile_meta", _I32, (slots, META_WORDS)), _ptr(num_splits, "num_splits", _I32, (b + 1,)),
        slots, _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(o_lat, "o_lat", _BF16, (b, s_q, h, D_LATENT)), _ptr(lse, "lse", (torch.float32,), (b, s_q, h)),
        _stream()), "mla_decode_paged_fp8")
    return o_lat, lse


def up_v(o_lat: torch.Tensor, w_uv: torch.Tensor, out=None):
    """o = o_lat @ W_UV per head, bf16 [b, s_q, h, 128]."""
    b, s_q, h, _ = o_lat.shape
    o = out if out is not None else torch.empty((b, s_q, h, D_NOPE), dtype=torch.bfloat16, device=o_lat.device)
    _check(load().mla_up_v(_ptr(o_lat, "o_lat", _BF16, (b, s_q, h, D_LATENT)),
                           _ptr(w_uv, "w_uv", _BF16, (h, D_LATENT, D_NOPE)),
                           _ptr(o, "o", _BF16, (b, s_q, h, D_NOPE)), b, s_q, h, _stream()), "mla_up_v")
    return o


def gather_pages(kv_cache, block_table, cache_seqlens, row_offsets, total_rows: int):
    """Rows of every cached token, in order, through the decode kernel's page loader."""
    b = cache_seqlens.numel()
    out = torch.empty((max(total_rows, 1), D_ROW), dtype=torch.bfloat16, device=kv_cache.device)
    _check(load().mla_gather_pages(_ptr(kv_cache, "kv_cache", _BF16), kv_cache.shape[0],
                                   _ptr(block_table, "block_table", _I32), block_table.shape[1],
                                   _ptr(cache_seqlens, "cache_seqlens", _I32), b,
                                   _ptr(row_offsets, "row_offsets", (torch.int64,), (b,)), _ptr(out, "out"),
                                   _stream()), "mla_gather_pages")
    return out[:total_rows]


def append_kv(new_rows, kv_cache, block_table, cache_seqlens):
    """Write new_rows [b, s_q, 576] into kv_cache in place: new row j of sequence b becomes token
    cache_seqlens[b] - s_q + j (the lengths count the new tokens)."""
    if new_rows.dim() != 3 or new_rows.shape[2] != D_ROW:
        raise MLAError(f"new_rows has shape {tuple(new_rows.shape)}, expected [b, s_q, {D_ROW}]")
    b, s_q = new_rows.shape[0], new_rows.shape[1]
    _check(load().mla_append_kv(_ptr(new_rows, "new_rows", _BF16), _ptr(kv_cache, "kv_cache", _BF16),
                                kv_cache.shape[0], _ptr(block_table, "block_table", _I32), block_table.shape[1],
                                _ptr(cache_seqlens, "cache_seqlens", _I32, (b,)), b, s_q, _stream()),
           "mla_append_kv")
    return kv_cache


def take_device_error() -> int:
    """MLA_DEVERR_* bits raised by kernels since the last call (synchronises)."""
    bits = _I(0)
    _check(load().mla_take_device_error(ctypes.byref(bits)), "mla_take_device_error")
    return bits.value
