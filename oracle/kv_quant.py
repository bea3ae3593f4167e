"""Quantised latent cache: 8-bit rows with one power-of-two scale per token.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The MLA engineering page ("DeepSeek-V3 Multi-head Latent Attention (MLA)
深度工程", section 7.2, quantised MLA) stores the compressed latent c^KV of each
token in 8 bits instead of 16, for half the cache memory; it fixes neither the
number format nor the scale. The reading taken here:

* The 512 latent values of a token are stored as OCP fp8 e4m3 ("e4m3fn": 1
  sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, no
  infinities, 0x7F/0xFF are NaN, largest finite value 448) after division by
  a per-token scale 2^e. The 64 decoupled-RoPE key values (section 3.1) are
  not part of c^KV and stay bf16.
* e is the smallest integer with max_i |c_i| <= 448 * 2^e, but not below
  -126 (so 2^e is a normal fp32 number); an all-zero row takes e = 0.
  Dividing by a power of two is exact, and the only rounding is the
  nearest-even rounding to e4m3.
* A page of 64 tokens is 41,216 bytes: 64 rows of 640 bytes (512 fp8 latent
  values, then the 64 bf16 key values as 128 bytes), then the 64 scales 2^e as
  fp32, in token order.

Dequantised values c = e4m3(code) * 2^e are exactly representable in bf16
(e4m3 has 3 mantissa bits), so a quantised cache is also a bf16 cache with
those values.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
PAGE = 64
D_LATENT = 512
D_ROPE = 64
ROW_BYTES = D_LATENT + 2 * D_ROPE          # 640
SCALES_OFFSET = PAGE * ROW_BYTES             # 40,960
PAGE_BYTES = SCALES_OFFSET + 4 * PAGE        # 41,216


def e4m3_value(code: int) -> float:
    """The value of an e4m3fn code (OCP definition): NaN for 0x7F and 0xFF."""
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def _rne_int(y: float) -> int:
    """Round a non-negative float to the nearest integer, ties to even."""
    f = math.floor(y)
    r = y - f
    if r > 0.5 or (r == 0.5 and f % 2 == 1):
        return int(f) + 1
    return int(f)


def e4m3_encode(x: float) -> int:
    """Nearest e4m3fn code to x, ties to the even code; |x| must not exceed 448.

    Below 2^-6 the format steps by 2^-9 (subnormals); in [2^E, 2^(E+1)) it
    steps by 2^(E-3). A result that rounds up to the next binade lands on the
    right code because the code is (E + 7) * 8 + mantissa steps.
    """
    a = abs(float(x))
    if a > E4M3_MAX:
        raise ValueError(f"{x} is outside the e4m3 range used here (|x| <= 448)")
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0
    if a < 2.0 ** -6:
        code = _rne_int(a * 2.0 ** 9)                     # 0 .. 8 (8 is 2^-6, the first normal)
    else:
        E = math.floor(math.log2(a))
        if 2.0 ** E > a:                                  # guard log2 rounding
            E -= 1
        elif 2.0 ** (E + 1) <= a:
            E += 1
        code = (E + 7) * 8 + _rne_int(a * 2.0 ** (3 - E)) - 8
    return sign | code


def scale_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e, at least -126; 0 for amax = 0."""
    if amax == 0.0:
        return 0
    mant, E = math.frexp(amax)         # amax = mant * 2^E, mant in [0.5, 1)
    mant, E = mant * 2.0, E - 1        # mant in [1, 2)
    e = E - 8 + (1 if mant > 1.75 else 0)
    return max(-126, e)


def quantize_row(row) -> tuple[np.ndarray, int, np.ndarray]:
    """One cache row (576 values, already bf16-exact) -> (512 e4m3 codes, e, 64 key values)."""
    row = np.asarray(row, dtype=np.float64)
    lat = row[:D_LATENT]
    e = scale_exponent(float(np.max(np.abs(lat))))
    codes = np.array([e4m3_encode(float(v) * 2.0 ** -e) for v in lat], dtype=np.uint8)
    return codes, e, row[D_LATENT:].copy()


def dequantize_row(codes, e: int, kpe) -> np.ndarray:
    """(codes, e, key values) -> the 576 values the quantised row stands for."""
    lat = np.array([e4m3_value(int(c)) for c in codes], dtype=np.float64) * 2.0 ** e
    return np.concatenate([lat, np.asarray(kpe, dtype=np.float64)])


# ---------------------------------------------------------------------------
# whole caches in the page format (vectorised forms of the two functions above)

_VALUES = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
_FINITE_POS = np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)  # codes 0x00 .. 0x7E


def _encode_array(y: np.ndarray) -> np.ndarray:
    """e4m3_encode over an array (|y| <= 448): nearest finite code, ties to the even code."""
    a = np.abs(y)
    idx = np.searchsorted(_FINITE_POS, a)             # first code whose value is >= a
    idx = np.clip(idx, 1, 126)
    lo, hi = _FINITE_POS[idx - 1], _FINITE_POS[idx]
    d_lo, d_hi = a - lo, hi - a
    code = np.where(d_lo < d_hi, idx - 1, idx)
    tie = d_lo == d_hi
    code = np.where(tie, np.where((idx - 1) % 2 == 0, idx - 1, idx), code)
    code = np.where(a == 0.0, 0, code)
    neg = np.signbit(y)
    return (code + np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_cache(kv_bf16_bits: np.ndarray) -> np.ndarray:
    """A bf16 paged cache [P, 64, 576] (bit patterns) -> the fp8 page format, uint8 [P, 41216]."""
    from mla_inputs import f32
    x = f32(kv_bf16_bits).astype(np.float64)                       # [P, 64, 576]
    P = x.shape[0]
    lat = x[:, :, :D_LATENT]
    amax = np.max(np.abs(lat), axis=2)
    exps = np.vectorize(scale_exponent, otypes=[np.int64])(amax) if P else np.zeros((0, PAGE), np.int64)
    scaled = lat * np.exp2(-exps.astype(np.float64))[:, :, None]
    codes = _encode_array(scaled)
    out = np.zeros((P, PAGE_BYTES), dtype=np.uint8)
    rows = out[:, :SCALES_OFFSET].reshape(P, PAGE, ROW_BYTES)
    rows[:, :, :D_LATENT] = codes
    rows[:, :, D_LATENT:] = np.ascontiguousarray(kv_bf16_bits[:, :, D_LATENT:]).view(np.uint8).reshape(P, PAGE, 2 * D_ROPE)
    scales = np.exp2(exps.astype(np.float64)).astype(np.float32)
    out[:, SCALES_OFFSET:] = scales.view(np.uint8).reshape(P, 4 * PAGE)
    return out


def dequantize_cache(pages: np.ndarray) -> np.ndarray:
    """The fp8 page format uint8 [P, 41216] -> the values it stands for, float64 [P, 64, 576]."""
    P = pages.shape[0]
    rows = pages[:, :SCALES_OFFSET].reshape(P, PAGE, ROW_BYTES)
    lat = _VALUES[rows[:, :, :D_LATENT]]
    scales = np.ascontiguousarray(pages[:, SCALES_OFFSET:]).view(np.float32).reshape(P, PAGE).astype(np.float64)
    kpe_bits = np.ascontiguousarray(rows[:, :, D_LATENT:]).view(np.uint16)
    kpe = (kpe_bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.concatenate([lat * scales[:, :, None], kpe], axis=2)


def append_rows_fp8(pages: np.ndarray, block_table: np.ndarray, seqlens: np.ndarray,
                    new_rows_bits: np.ndarray) -> np.ndarray:
    """The fp8 cache after quantising and storing the step's new rows (a copy).

    New row j of sequence b is token t = L_b - s_q + j (the lengths count the
    new tokens), at page block_table[b, t // 64], slot t % 64: its 640 row
    bytes and its scale are written. Rows with a negative token index, a token
    past the block table or a page id outside the cache are skipped.
    """
    from mla_inputs import f32
    out = pages.copy()
    b_count, s_q = new_rows_bits.shape[0], new_rows_bits.shape[1]
    for b in range(b_count):
        for j in range(s_q):
            t = int(seqlens[b]) - s_q + j
            if t < 0 or t // PAGE >= block_table.shape[1]:
                continue
            pid = int(block_table[b, t // PAGE])
            if not 0 <= pid < pages.shape[0]:
                continue
            codes, e, _ = quantize_row(f32(new_rows_bits[b, j]))
            slot = t % PAGE
            row = out[pid, slot * ROW_BYTES:(slot + 1) * ROW_BYTES]
            row[:D_LATENT] = codes
            row[D_LATENT:] = np.ascontiguousarray(new_rows_bits[b, j, D_LATENT:]).view(np.uint8)
            out[pid, SCALES_OFFSET + 4 * slot:SCALES_OFFSET + 4 * slot + 4] = \
                np.array([2.0 ** e], dtype=np.float32).view(np.uint8)
    return out
