"""Pins of the quantised-cache oracle (oracle/kv_quant.py) against things other than itself:
hand-worked codes of the e4m3 definition, brute-force nearest-value search, the defining
inequality of the scale exponent, round trips and a hand-quantised row."""
import math

import numpy as np
import pytest

from mla_inputs import bf16_bits, f32, make_inputs
from oracle import kv_quant as Q

# Hand-worked e4m3fn codes: sign | exponent (bias 7) << 3 | mantissa.
HAND = [
    (0.0, 0x00), (2.0 ** -9, 0x01), (7 * 2.0 ** -9, 0x07), (2.0 ** -6, 0x08), (0.5, 0x30), (1.0, 0x38),
    (1.125, 0x39), (1.75, 0x3E), (2.0, 0x40), (3.0, 0x44), (240.0, 0x77), (256.0, 0x78), (448.0, 0x7E),
    (-1.0, 0xB8), (-2.0, 0xC0), (-448.0, 0xFE),
]


@pytest.mark.parametrize("x,code", HAND)
def test_hand_worked_codes(x, code):
    assert Q.e4m3_encode(x) == code
    assert Q.e4m3_value(code) == x


def test_nan_codes_and_table_shape():
    assert math.isnan(Q.e4m3_value(0x7F)) and math.isnan(Q.e4m3_value(0xFF))
    vals = [Q.e4m3_value(c) for c in range(127)]
    assert all(a < b for a, b in zip(vals, vals[1:]))  # codes 0..126 are increasing
    assert vals[-1] == 448.0 and len(set(vals)) == 127


def test_every_finite_code_round_trips():
    for c in range(256):
        v = Q.e4m3_value(c)
        if math.isnan(v):
            continue
        assert Q.e4m3_encode(v) == c, (c, v)


def _brute_nearest(x):
    """The finite code whose value is nearest to x; on a tie, the even code (by search, not formula)."""
    best = None
    for c in range(256):
        v = Q.e4m3_value(c)
        if math.isnan(v) or (v == 0.0 and c == 0x80):
            continue
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    c = best[1]
    if Q.e4m3_value(c) == 0.0 and math.copysign(1.0, x) < 0:
        c = 0x80
    return c


def test_encode_is_nearest_even_by_brute_force():
    rng = np.random.default_rng(1)
    xs = list(rng.uniform(-448, 448, 300)) + list(rng.standard_normal(300) * 0.01)
    vals = [Q.e4m3_value(c) for c in range(127)]
    for a, b in zip(vals, vals[1:]):  # every midpoint (a tie) and its neighbours
        mid = (a + b) / 2
        xs += [mid, -mid, np.nextafter(mid, 1e9), np.nextafter(mid, -1e9)]
    for x in xs:
        assert Q.e4m3_encode(float(x)) == _brute_nearest(float(x)), x
    arr = np.array(xs, dtype=np.float64)
    assert np.array_equal(Q._encode_array(arr), np.array([Q.e4m3_encode(float(x)) for x in xs], dtype=np.uint8))


def test_hand_worked_ties():
    assert Q.e4m3_encode(136.0) == 0x70    # between 128 (0x70, even) and 144: the even code
    assert Q.e4m3_encode(152.0) == 0x72    # between 144 (0x71) and 160 (0x72, even)
    assert Q.e4m3_encode(2.0 ** -10) == 0x00  # half of the smallest subnormal rounds to 0 (even)
    assert Q.e4m3_encode(3 * 2.0 ** -10) == 0x02  # between 0x01 and 0x02: the even code


def test_scale_exponent_is_the_smallest_that_fits():
    rng = np.random.default_rng(2)
    amaxes = [0.0, 1.0, 1.75, 1.7500001, 2.0, 448.0, 449.0, 3.0, 0.001, 1e-30, 1e30] + \
        list(np.exp(rng.uniform(-20, 20, 200)))
    for a in amaxes:
        e = Q.scale_exponent(float(a))
        if a == 0.0:
            assert e == 0
            continue
        # brute force over integers: the smallest e with a <= 448 * 2^e, clipped at -126
        e_bf = next(k for k in range(-200, 200) if a <= 448.0 * 2.0 ** k)
        assert e == max(e_bf, -126), (a, e, e_bf)


def test_hand_quantised_row():
    row = np.zeros(576)
    row[:5] = [1.0, -0.5, 3.0, 1.0625, 1.1875]
    row[512:515] = [7.0, -1.5, 0.25]
    codes, e, kpe = Q.quantize_row(row)
    # amax 3 = 1.5 * 2^1 -> e = 1 - 8 = -7: values are scaled by 128
    assert e == -7
    assert list(codes[:5]) == [0x70, 0xE8, 0x7C, 0x70, 0x72]  # 128, -64, 384, 136 -> 128, 152 -> 160
    assert not codes[5:].any()
    assert np.array_equal(kpe, row[512:])
    back = Q.dequantize_row(codes, e, kpe)
    assert list(back[:5]) == [1.0, -0.5, 3.0, 1.0, 1.25]


def test_round_trip_bound_and_bf16_exactness():
    inp = make_inputs("tiny", seed=3)
    x = f32(inp.kv_cache).astype(np.float64)
    pages = Q.quantize_cache(inp.kv_cache)
    y = Q.dequantize_cache(pages)
    lat_x, lat_y = x[:, :, :512], y[:, :, :512]
    amax = np.abs(lat_x).max(axis=2, keepdims=True)
    # normal e4m3 values carry 3 mantissa bits: at most half a step (2^-4 relative) away;
    # below the subnormal threshold the step is 2^-9 of the scale
    scale = np.exp2([[Q.scale_exponent(float(a)) for a in r] for r in amax[:, :, 0]])[:, :, None]
    bound = np.maximum(np.abs(lat_x) * 2.0 ** -4, scale * 2.0 ** -10)
    assert (np.abs(lat_x - lat_y) <= bound).all()
    assert np.array_equal(y[:, :, 512:], x[:, :, 512:])               # the key part is kept exactly
    assert np.array_equal(f32(bf16_bits(y.astype(np.float32))), y.astype(np.float32))  # bf16-exact
    # every row's largest latent value lands in [224, 448] (above 224 before rounding to the 16-step grid)
    top = np.abs(lat_y).max(axis=2) / scale[:, :, 0]
    assert ((top >= 224) & (top <= 448)).all()


def test_page_layout_by_hand():
    inp = make_inputs("tiny", seed=4)
    pages = Q.quantize_cache(inp.kv_cache)
    assert pages.shape == (inp.num_pages, 41216)
    p, s = 1, 5
    codes, e, _ = Q.quantize_row(f32(inp.kv_cache[p, s]))
    row = pages[p, s * 640:(s + 1) * 640]
    assert np.array_equal(row[:512], codes)
    assert np.array_equal(row[512:].view(np.uint16), inp.kv_cache[p, s, 512:])
    assert pages[p, 40960 + 4 * s:40960 + 4 * s + 4].view(np.float32)[0] == 2.0 ** e


def test_append_fp8_matches_quantising_the_appended_bf16_cache():
    from mla_inputs import make_new_rows
    from oracle import mla_oracle as O
    inp = make_inputs("tiny", seed=5, seqlens=[37, 100, 64], s_q=2)
    new = make_new_rows(inp, seed=6)
    pages = Q.quantize_cache(inp.kv_cache)
    got = Q.append_rows_fp8(pages, inp.block_table, inp.seqlens, new)
    want = Q.quantize_cache(O.append_rows(inp.kv_cache, inp.block_table, inp.seqlens, new))
    assert np.array_equal(got, want)
    assert not np.array_equal(got, pages)


# ---------------------------------------------------------------------------
# planted mistakes: each must make one of the pins above fail

def _rne_half_up(y):
    return int(math.floor(y + 0.5))


def _value_bias8(code):
    sign = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    return sign * ((m / 8.0) * 2.0 ** -7 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 8))


def _scale_no_mantissa_check(amax):
    if amax == 0.0:
        return 0
    mant, E = math.frexp(amax)
    return max(-126, E - 1 - 8)


def _scale_always_up(amax):
    if amax == 0.0:
        return 0
    mant, E = math.frexp(amax)
    return max(-126, E - 1 - 7)


def _encode_array_ties_up(y):
    a = np.abs(y)
    idx = np.clip(np.searchsorted(Q._FINITE_POS, a), 1, 126)
    lo, hi = Q._FINITE_POS[idx - 1], Q._FINITE_POS[idx]
    code = np.where(a - lo < hi - a, idx - 1, idx)
    code = np.where(a == 0.0, 0, code)
    return (code + np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


KQ_MUTATIONS = {
    "encode_rounds_half_up": ("_rne_int", _rne_half_up),
    "value_bias_8": ("e4m3_value", _value_bias8),
    "scale_ignores_mantissa": ("scale_exponent", _scale_no_mantissa_check),
    "scale_one_binade_high": ("scale_exponent", _scale_always_up),
    "array_encode_ties_up": ("_encode_array", _encode_array_ties_up),
}

KQ_PINS = [test_every_finite_code_round_trips, test_hand_worked_ties, test_scale_exponent_is_the_smallest_that_fits,
           test_hand_quantised_row, test_encode_is_nearest_even_by_brute_force,
           test_round_trip_bound_and_bf16_exactness, test_page_layout_by_hand,
           test_append_fp8_matches_quantising_the_appended_bf16_cache]


@pytest.mark.parametrize("name", sorted(KQ_MUTATIONS))
def test_kv_quant_mutation_is_caught(name, monkeypatch):
    attr, bad = KQ_MUTATIONS[name]
    monkeypatch.setattr(Q, attr, bad)
    if attr == "e4m3_value":  # the vectorised tables are built from it at import
        monkeypatch.setattr(Q, "_VALUES", np.array([bad(c) for c in range(256)]))
        monkeypatch.setattr(Q, "_FINITE_POS", np.array([bad(c) for c in range(127)]))
    caught = False
    for pin in [lambda: [test_hand_worked_codes(x, c) for x, c in HAND]] + KQ_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts as caught
            caught = True
            break
    assert caught, f"mutation {name} slipped past every pin"
