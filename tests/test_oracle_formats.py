"""Pins of the oracle's format machinery (tier 0) against facts fixed outside it.

* constants printed on the pages (tests/golden/format_constants.json);
* library routines: numpy's IEEE binary16 conversion and torch's float8
  conversions (round to nearest even, non-saturating);
* closed forms and exhaustive enumeration of all codes.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import BF16, E4M3, E5M2, FP16, Val
from oracle.cast import cast_element
from oracle.formats import pow2


def _val_to_float(v):
    if v.kind == "nan":
        return math.nan
    if v.kind == "inf":
        return -math.inf if v.neg else math.inf
    f = float(v.mag)
    return -f if v.neg else f


def _same_float(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


# -- FP16: the generic machinery at the printed FP16 parameters ---------------

def test_fp16_printed_constants(consts):
    g = consts["fp16"]
    assert (FP16.ebits, FP16.mbits) == (g["exponent_bits"], g["mantissa_bits"])
    assert FP16.maxval == g["max"] == pow2(15) * (2 - pow2(-10))
    assert FP16.decode(0x7BFF).mag == g["max"]
    assert FP16.decode(0x0400).mag == pow2(g["min_normal_log2"])
    assert FP16.decode(0x0001).mag == pow2(g["min_subnormal_log2"])
    assert FP16.min_subnormal == pow2(g["min_subnormal_log2"])


def test_fp16_decode_matches_numpy_all_codes():
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    for code in range(65536):
        assert _same_float(_val_to_float(FP16.decode(code)), float(ref[code])), hex(code)


def test_fp16_encode_matches_numpy_on_all_bf16_values():
    """Round-to-nearest-even with IEEE overflow, at FP16's parameters, against
    numpy's binary64 -> binary16 conversion, for every bf16 input value."""
    vals = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = vals.astype(np.float16).view(np.uint16)
    for i, x in enumerate(vals.tolist()):
        code = FP16.encode(Val.of(x), saturate=False)
        if math.isnan(x):
            assert FP16.decode(code).kind == "nan"
        else:
            assert code == int(ref[i]), (hex(i), x)


# -- BF16 -----------------------------------------------------------------------

def test_bf16_decode_matches_numpy_and_printed_range(consts):
    g = consts["bf16"]
    assert (BF16.ebits, BF16.mbits) == (g["exponent_bits"], g["mantissa_bits"])
    ref = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    for code in range(65536):
        assert _same_float(_val_to_float(BF16.decode(code)), float(ref[code])), hex(code)
    assert abs(float(BF16.maxval) / g["max_approx"] - 1) < 0.01


# -- FP8 layouts ------------------------------------------------------------------

def _brute_decode(code, ebits, mbits, bias, scheme):
    """An independent decoder for candidate 8-bit layouts: 'ieee' (all-ones
    exponent = Inf/NaN), 'fn' (only all-ones exponent+mantissa = NaN),
    'fnuz' (no negative zero: 0x80 is the only NaN, no Inf)."""
    s = code >> 7
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if scheme == "fnuz" and code == 0x80:
        return "nan"
    if scheme == "ieee" and e == (1 << ebits) - 1:
        return "inf" if m == 0 else "nan"
    if scheme == "fn" and e == (1 << ebits) - 1 and m == (1 << mbits) - 1:
        return "nan"
    if e == 0:
        mag = Fraction(m, 1 << mbits) * pow2(1 - bias)
    else:
        mag = (1 + Fraction(m, 1 << mbits)) * pow2(e - bias)
    return (-1 if s else 1, mag)


@pytest.mark.parametrize("name,fmt", [("e4m3", E4M3), ("e5m2", E5M2)])
def test_fp8_layout_forced_by_printed_max(consts, name, fmt):
    """Among bias/special-value layouts with the printed bit counts, exactly
    one has the printed largest value and a negative zero -- the oracle's."""
    g = consts[name]
    eb, mb = g["exponent_bits"], g["mantissa_bits"]
    matches = []
    for bias in range((1 << (eb - 1)) - 3, (1 << (eb - 1)) + 3):
        for scheme in ("ieee", "fn", "fnuz"):
            vals = [_brute_decode(c, eb, mb, bias, scheme) for c in range(256)]
            finite = [v for v in vals if isinstance(v, tuple)]
            mx = max(m for _, m in finite)
            has_neg_zero = any(s < 0 and m == 0 for s, m in finite)
            if mx == g["max"] and has_neg_zero == g["has_negative_zero"]:
                matches.append((bias, scheme))
    want = (fmt.bias, "ieee" if fmt.specials == "ieee" else "fn")
    assert matches == [want]
    assert fmt.maxval == g["max"]


@pytest.mark.parametrize("fmt,tdt", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_fp8_decode_matches_torch_all_codes(fmt, tdt):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(tdt).to(torch.float64).tolist()
    for code in range(256):
        assert _same_float(_val_to_float(fmt.decode(code)), ref[code]), hex(code)


def test_fp8_code_tables():
    """Closed-form counts of the two tables (256 codes each)."""
    def census(fmt):
        vals = [fmt.decode(c) for c in range(256)]
        fin = [v for v in vals if v.kind == "num"]
        return (len(fin), len({v.signed for v in fin}),
                sum(v.kind == "nan" for v in vals), sum(v.kind == "inf" for v in vals))
    assert census(E4M3) == (254, 253, 2, 0)
    assert census(E5M2) == (248, 247, 6, 2)
    assert E4M3.decode(0x08).mag == pow2(-6) and E4M3.decode(0x07).mag < pow2(-6)
    assert E4M3.decode(0x01).mag == pow2(-9) and E4M3.max_code() == 0x7E
    assert E5M2.decode(0x04).mag == pow2(-14) and E5M2.decode(0x03).mag < pow2(-14)
    assert E5M2.decode(0x01).mag == pow2(-16) and E5M2.max_code() == 0x7B
    assert E4M3.decode(0x80).neg and E4M3.decode(0x80).mag == 0
    assert E5M2.decode(0x80).neg and E5M2.decode(0x80).mag == 0


def _torch_cast(values_f32, tdt):
    return torch.tensor(values_f32, dtype=torch.float32).to(tdt).view(torch.uint8).tolist()


@pytest.mark.parametrize("fmt,tdt", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_fp8_encode_matches_torch_on_all_bf16_values_in_range(fmt, tdt):
    """torch's float32 -> float8 cast rounds to nearest even (and does not
    saturate): on every bf16 value with |x| <= M_F the oracle must agree."""
    vals = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= float(fmt.maxval))
    vals = vals[keep]
    ref = _torch_cast(vals.tolist(), tdt)
    for x, r in zip(vals.tolist(), ref):
        code, clip, uf, nf = cast_element(fmt, Val.of(x), 0)
        assert code == r, (x, hex(code), hex(r))
        assert not clip and not nf
        assert uf == (x != 0 and (code & 0x7F) == 0)


@pytest.mark.parametrize("fmt,tdt", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)])
def test_fp8_encode_matches_torch_at_midpoints(fmt, tdt):
    """Every midpoint between adjacent finite codes, and the fp32 neighbours
    of each midpoint: the tie and both sides of it."""
    mags = sorted({fmt.decode(c).mag for c in range(128) if fmt.decode(c).kind == "num"})
    xs = []
    for lo, hi in zip(mags, mags[1:]):
        mid = np.float32(float((lo + hi) / 2))
        assert Fraction(float(mid)) == (lo + hi) / 2
        xs += [float(np.nextafter(mid, np.float32(0))), float(mid),
               float(np.nextafter(mid, np.float32(np.inf)))]
    xs += [-x for x in xs]
    ref = _torch_cast(xs, tdt)
    for x, r in zip(xs, ref):
        assert cast_element(fmt, Val.of(x), 0)[0] == r, x


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_saturation_and_special_inputs(fmt):
    M = fmt.maxval
    for x in (float(M) * 1.0001, float(M) * 2, 1e30, 3.0e38):
        for s in (1, -1):
            code, clip, uf, nf = cast_element(fmt, Val.of(s * x), 0)
            assert code == fmt.max_code(s < 0) and clip and not uf and not nf
    code, clip, uf, nf = cast_element(fmt, Val.of(float(M)), 0)
    assert code == fmt.max_code() and not clip
    assert cast_element(fmt, Val.of(math.inf), 0) == (fmt.max_code(False), False, False, True)
    assert cast_element(fmt, Val.of(-math.inf), 0) == (fmt.max_code(True), False, False, True)
    assert cast_element(fmt, Val("nan", True, Fraction(0)), 0) == (0x7F, False, False, True)
    assert cast_element(fmt, Val.of(-0.0), 0) == (0x80, False, False, False)
    assert cast_element(fmt, Val.of(0.0), 0) == (0x00, False, False, False)


@pytest.mark.parametrize("fmt", [E4M3, E5M2])
def test_round_trip_every_code(fmt):
    for code in range(256):
        v = fmt.decode(code)
        out = cast_element(fmt, v, 0)[0]
        if v.kind == "nan":
            assert out == 0x7F
        elif v.kind == "inf":
            assert out == fmt.max_code(v.neg)
        else:
            assert out == code


def test_underflow_and_saturation_edges():
    """E4M3: |y| <= 2^-10 rounds to zero (the tie goes to even zero);
    (448, 464] rounds to 448 (464 is a tie to even 448).  E5M2: |y| <= 2^-17
    underflows; 61440 is a tie that would round to 65536, so it saturates."""
    def c(fmt, x):
        return cast_element(fmt, Val.of(x), 0)
    assert c(E4M3, 2.0 ** -10)[0] == 0 and c(E4M3, 2.0 ** -10)[2]
    assert c(E4M3, float(np.nextafter(np.float32(2.0 ** -10), np.float32(1))))[0] == 1
    assert c(E4M3, -(2.0 ** -10))[0] == 0x80 and c(E4M3, -(2.0 ** -10))[2]
    assert c(E4M3, 464.0)[0] == 0x7E and c(E4M3, 464.0)[1]
    assert c(E4M3, 460.0)[0] == 0x7E and c(E4M3, 460.0)[1]
    assert c(E4M3, 440.0)[0] == 0x7E and not c(E4M3, 440.0)[1]      # tie 416|448 -> even 448
    assert c(E5M2, 2.0 ** -17)[0] == 0 and c(E5M2, 2.0 ** -17)[2]
    assert c(E5M2, float(np.nextafter(np.float32(2.0 ** -17), np.float32(1))))[0] == 1
    assert c(E5M2, 61440.0)[0] == 0x7B and c(E5M2, 61440.0)[1]
    assert c(E5M2, 61439.0)[0] == 0x7B and c(E5M2, 61439.0)[1]
