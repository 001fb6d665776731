"""All 65,536 pairs of 8-bit values, multiplied and added, per format
([Drift, "First, catching myself"]: two implementations compared on every
value and every pair, signed zero included).

Tier 0 (exact rationals with an explicit sign bit, IEEE sign rules written
out) is compared with tier 1 (binary64 arithmetic, exact for these operands,
whose signed-zero behaviour is IEEE's), and both with torch's float8 cast
where torch's cast is defined the same way (results within range).
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import E4M3, E5M2, Val
from oracle import bulk
from oracle.cast import cast_element


def _mul(a: Val, b: Val) -> Val:
    if a.kind == "nan" or b.kind == "nan":
        return Val("nan", False, Fraction(0))
    neg = a.neg != b.neg
    if a.kind == "inf" or b.kind == "inf":
        other = b if a.kind == "inf" else a
        if other.kind == "num" and other.mag == 0:
            return Val("nan", False, Fraction(0))
        return Val("inf", neg, Fraction(0))
    return Val.num(neg, a.mag * b.mag)


def _add(a: Val, b: Val) -> Val:
    if a.kind == "nan" or b.kind == "nan":
        return Val("nan", False, Fraction(0))
    if a.kind == "inf" and b.kind == "inf":
        return Val("inf", a.neg, Fraction(0)) if a.neg == b.neg else Val("nan", False, Fraction(0))
    if a.kind == "inf" or b.kind == "inf":
        return a if a.kind == "inf" else b
    s = a.signed + b.signed
    if s == 0:
        # exact zero sum under round-to-nearest: -0 only for (-0) + (-0)
        return Val.num(a.neg and b.neg and a.mag == 0 and b.mag == 0, 0)
    return Val.of(s)


def _tier0_pairs(fmt, op):
    dec = [fmt.decode(c) for c in range(256)]
    out = np.empty((256, 256), dtype=np.uint8)
    for i in range(256):
        for j in range(256):
            out[i, j] = cast_element(fmt, op(dec[i], dec[j]), 0)[0]
    return out


@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("opname", ["mul", "add"])
def test_all_pairs_tier0_vs_tier1(fmt, opname, consts):
    assert 256 * 256 == consts["pairs_per_8bit_format"]
    t0 = _tier0_pairs(fmt, _mul if opname == "mul" else _add)
    d = bulk.decode_table(fmt)
    a, b = np.meshgrid(d, d, indexing="ij")
    with np.errstate(invalid="ignore"):
        r = a * b if opname == "mul" else a + b
    t1 = bulk.cast_f64(fmt, r, 0)[0]
    bad = np.argwhere(t0 != t1)
    assert bad.size == 0, [(hex(i), hex(j), hex(t0[i, j]), hex(t1[i, j])) for i, j in bad[:10]]


@pytest.mark.parametrize("fmt,tdt", [(E4M3, torch.float8_e4m3fn), (E5M2, torch.float8_e5m2)],
                         ids=["e4m3", "e5m2"])
@pytest.mark.parametrize("opname", ["mul", "add"])
def test_pairs_vs_torch_cast(fmt, tdt, opname):
    """Pairs whose exact result is an fp32 value within range: torch's
    float32 -> float8 cast (round to nearest even) must give the same code."""
    d = bulk.decode_table(fmt)
    a, b = np.meshgrid(d, d, indexing="ij")
    with np.errstate(invalid="ignore", over="ignore"):
        r64 = a * b if opname == "mul" else a + b
        r32 = r64.astype(np.float32)
    ok = np.isfinite(r64) & (r32.astype(np.float64) == r64) & (np.abs(r64) <= float(fmt.maxval))
    ref = torch.from_numpy(r32[ok]).to(tdt).view(torch.uint8).numpy()
    mine = bulk.cast_f64(fmt, r64[ok], 0)[0]
    assert np.array_equal(mine, ref)
    # the pairs compared cover most of the table
    assert ok.sum() > 0.5 * ok.size


@pytest.mark.parametrize("fmt,expected", [(E4M3, 506), (E5M2, 494)], ids=["e4m3", "e5m2"])
def test_negative_zero_products(fmt, expected):
    """Finite pairs whose exact product is -0: one factor is a zero and the
    signs differ.  With z+ = 1 (+0), n = finite nonzero codes per sign, the
    count is 2 * (n + 1) + 2 * n (closed form of the IEEE sign rule)."""
    dec = [fmt.decode(c) for c in range(256)]
    n_per_sign = sum(1 for v in dec if v.kind == "num" and v.mag != 0 and not v.neg)
    assert 2 * (n_per_sign + 1) + 2 * n_per_sign == expected
    count = 0
    for a in dec:
        for b in dec:
            if a.kind == "num" and b.kind == "num":
                p = _mul(a, b)
                if p.mag == 0 and p.neg:
                    assert cast_element(fmt, p, 0)[0] == 0x80
                    count += 1
    assert count == expected


def test_signed_zero_sum_rules():
    z, nz, one, mone = Val.of(0.0), Val.of(-0.0), Val.of(1.0), Val.of(-1.0)
    assert _add(nz, nz).neg and not _add(z, nz).neg and not _add(one, mone).neg
    assert math.copysign(1.0, -0.0 + -0.0) < 0 and math.copysign(1.0, 1.0 + -1.0) > 0
