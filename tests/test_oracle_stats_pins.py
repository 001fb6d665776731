"""Pins of the oracle's error statistics and of the value a code stands for,
against values fixed outside the oracle.

The statistics measure the size of the change the cast makes to a tensor
and, apart from it, the change's direction (page "what actually breaks low precision
training", section "What the measurements said"): over finite elements,
with xhat = decode(q) * 2^-K and e = xhat - x, the sums of e, |e|, e^2,
sign(x) e, x e and x^2.  Pinned here by:

* hand-worked elements (tests/golden/stats_hand.json): the code, the
  represented value and all six terms of each, clips, ties, underflows, a
  subnormal rounding up, a signed zero, per-tensor and MX exponents, in both
  formats; and their sums per format, rounded once to binary64 -- for tier 0
  (exact rationals) and tier 1 (vectorised binary64) separately;
* hand-worked dequantised bf16 patterns (tests/golden/dequant_hand.json),
  including the direction of the scale (2^-K, and 2^X for an MX block) and
  bf16's subnormal and overflow edges;
* a property every in-range element must have: the represented value is
  within half a grid step of x (the step from the format's printed layout);
* a closed form for the 4096 x 4096 bf16 tanh(N(0, 1.5)) workload's
  sign-aligned bias, kept fraction and relative RMS error under the OCP, +1
  and ceil block rules (scipy's normal distribution for how often each bf16
  value occurs, torch's float8 conversion for the rounding), against the
  oracle's sums on a 4M-element sample.

The last test plants plausible mistakes in the oracle (a flipped error sign,
x e computed as xhat e, a dropped absolute value, the square of the wrong
value, sign(xhat) for sign(x), the scale applied the wrong way) and checks
that the pins above fail on each.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle import E4M3, E5M2, Val, bulk
from oracle import cast as t0
from tests.conftest import load_golden
import workloads

FMT = {"e4m3": E4M3, "e5m2": E5M2}
STATS = load_golden("stats_hand.json")
DEQ = load_golden("dequant_hand.json")


def _val(s: str) -> Val:
    """A tier-0 value from a golden string, keeping the sign of '-0'."""
    f = Fraction(s)
    return Val.num(s.strip().startswith("-"), abs(f))


def _f64(s: str) -> float:
    v = _val(s)
    return -float(v.mag) if v.neg else float(v.mag)


# -- the pins, as functions (the planted-mistake test runs them again) --------

def check_terms_tier0():
    for c in STATS["cases"]:
        fmt, K, v = FMT[c["fmt"]], c["K"], _val(c["x"])
        code, clip, uf, nf = t0.cast_element(fmt, v, K)
        assert code == int(c["code"], 16), c["id"]
        xh = t0.represented(fmt, code, K)
        want = _val(c["xhat"])
        assert (xh.neg, xh.mag) == (want.neg, want.mag), c["id"]
        got = t0.stats_terms(v.signed, xh.signed)
        assert [Fraction(g) for g in got] == [Fraction(t) for t in c["terms"]], c["id"]


def check_terms_tier1():
    for c in STATS["cases"]:
        fmt, K = FMT[c["fmt"]], c["K"]
        x = np.array([_f64(c["x"])])
        codes = bulk.cast_f64(fmt, x, K)[0]
        assert int(codes[0]) == int(c["code"], 16), c["id"]
        xh = bulk.represented_f64(fmt, codes, K)
        assert xh[0] == _f64(c["xhat"]) and np.signbit(xh[0]) == np.signbit(_f64(c["xhat"])), c["id"]
        got = [float(t[0]) for t in bulk.stats_terms_f64(x, xh)]
        assert got == [float(Fraction(t)) for t in c["terms"]], c["id"]


def check_sums():
    for name, fmt in FMT.items():
        cases = [c for c in STATS["cases"] if c["fmt"] == name]
        want = {k: float(Fraction(v)) for k, v in zip(t0.STAT_KEYS, STATS["sums"][name])}
        vals = [_val(c["x"]) for c in cases]
        codes = [int(c["code"], 16) for c in cases]
        Ks = [c["K"] for c in cases]
        assert t0.stats(fmt, vals, codes, Ks) == want, name
        x = np.array([_f64(c["x"]) for c in cases])
        got1 = bulk.stats_f64(fmt, x, np.array(codes, dtype=np.uint8), np.array(Ks))
        assert got1 == want, name


def check_dequant():
    for c in DEQ["cases"]:
        fmt, code, K, want = FMT[c["fmt"]], int(c["code"], 16), c["K"], int(c["bf16"], 16)
        assert t0.dequant_bf16(fmt, code, K) == want, c
        assert int(bulk.dequant_bf16_f64(fmt, np.array([code], dtype=np.uint8), K)[0]) == want, c


PINS = (check_terms_tier0, check_terms_tier1, check_sums, check_dequant)


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_hand_worked_pins(pin):
    pin()


# -- the represented value is the nearest grid point ---------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_round_trip_within_half_a_step(fmt):
    """For every finite x whose scaled value y = x 2^K does not clip,
    |xhat - x| <= half the grid step at y, with the step read off the
    format's layout (mantissa bits p, smallest normal 2^emin, subnormal step
    2^(emin - p)); a distance of exactly half a step only on a code whose
    last mantissa bit is 0 (ties to even)."""
    rng = np.random.default_rng(61)
    n = 200000
    x = workloads.mixed_magnitude_fp32(n, 62, -40, 40).astype(np.float64)
    K = rng.integers(-30, 30, n)
    # plus every midpoint between neighbouring grid values below the maximum,
    # from the layout (normal binades emin..emax, subnormals below), at
    # random K and signs: the ties
    m = np.arange(2 ** fmt.mbits)
    mids = [np.ldexp(m + 0.5, fmt.emin - fmt.mbits)]
    mids += [np.ldexp(2 ** fmt.mbits + m + 0.5, b - fmt.mbits) for b in range(fmt.emin, fmt.emax + 1)]
    mids = np.concatenate(mids)
    mids = mids[mids < float(fmt.maxval)]
    Km = rng.integers(-30, 30, mids.size)
    x = np.concatenate([x, np.ldexp(mids, -Km) * rng.choice([-1.0, 1.0], mids.size)])
    K = np.concatenate([K, Km])
    y = np.abs(np.ldexp(x, K))
    keep = y <= float(fmt.maxval)
    x, K, y = x[keep], K[keep], y[keep]
    codes = bulk.cast_f64(fmt, x, K)[0]
    xh = bulk.represented_f64(fmt, codes, K)
    _, ex = np.frexp(y)
    binade = np.maximum(ex.astype(np.int64) - 1, fmt.emin)
    step = np.ldexp(1.0, binade - fmt.mbits - K)              # in x's units
    dist = np.abs(xh - x)
    assert np.all(dist <= step / 2)
    tie = dist == step / 2
    assert np.all((codes[tie] & 1) == 0)
    assert tie.any() and (dist < step / 2).any()


# -- the tanh workload: bias and kept fraction in closed form ------------------

def tanh_expected(rule: str, sd: float = 1.5, block: int = 32):
    """Expected per-element sign-aligned error, kept fraction 1 + E[x e] / E[x^2]
    and relative RMS error of bf16 tanh(N(0, sd)) under an MX block rule
    (E4M3, blocks of 32).  Every bf16 value w in (0, 1] occurs with
    probability P(w) = P(tanh(z) rounds to +-w), from scipy's normal
    distribution; the value is rounded at the block's exponent K with torch's
    float8_e4m3fn conversion (nearest even), and clipped to 448 past it.  A
    block's exponent depends on its largest element only (blocks with a
    largest element below 1/2 have probability ~1e-17 and are left out):
    OCP: K = 8 if the block holds an exact 1.0, else 9;  +1: one less;
    ceil: K = 8 if the block's largest element exceeds 0.875, else 9."""
    pat = np.arange(1, 0x3F81, dtype=np.uint32)                 # bf16 patterns of (0, 1]
    w = (pat << np.uint32(16)).view(np.float32).astype(np.float64)
    below = np.where(pat > 1, ((pat - 1) << np.uint32(16)).view(np.float32).astype(np.float64), 0.0)
    above = ((pat + 1) << np.uint32(16)).view(np.float32).astype(np.float64)
    lo, hi = (w + below) / 2, np.minimum((w + above) / 2, 1.0)
    with np.errstate(divide="ignore"):
        P = 2 * (norm.cdf(np.arctanh(hi) / sd) - norm.cdf(np.arctanh(lo) / sd))
    P[-1] = 2 * norm.sf(np.arctanh(lo[-1]) / sd)                # w = 1.0: every t >= 1 - 2^-9

    def xhat(K):
        y = w * 2.0 ** K
        r = torch.from_numpy(y).to(torch.float8_e4m3fn).to(torch.float64).numpy()
        return np.where(y > 448.0, 448.0, r) * 2.0 ** -K

    if rule in ("ocp", "plus1"):
        p_other = 1 - (1 - P[-1]) ** (block - 1)                # another element is 1.0
        pa = np.where(w == 1.0, 1.0, p_other)
        Ka, Kb = (8, 9) if rule == "ocp" else (7, 8)
    else:
        p_big = P[w > 0.875].sum()
        pa = np.where(w > 0.875, 1.0, 1 - (1 - p_big) ** (block - 1))
        Ka, Kb = 8, 9
    da, db = xhat(Ka) - w, xhat(Kb) - w
    d = pa * da + (1 - pa) * db
    ex2 = np.sum(P * w * w)
    return dict(sign_aligned=float(np.sum(P * d)), kept=float(1 + np.sum(P * w * d) / ex2),
                rel_rms=float(math.sqrt(np.sum(P * (pa * da ** 2 + (1 - pa) * db ** 2)) / ex2)),
                p_total=float(P.sum()))


# Bands: the sample's statistical spread (4M elements, blocks of 32) is a few
# 1e-5 on the OCP bias and kept fraction and a few 1e-6 under +1 and ceil; the
# closed form drops the double rounding fp64 -> fp32 -> bf16 of the inputs
# (effect ~2^-24 relative per boundary) and blocks whose largest element is
# below 1/2.  A flipped error sign moves the bias by 2.6e-2 (OCP) / 2.3e-3;
# x e taken as xhat e moves the kept fraction by the squared relative RMS
# error, 2.7e-3 (OCP) / 4.4e-4.
TANH_BANDS = {"ocp": (3e-4, 4e-4, 1e-3), "plus1": (3e-5, 3e-5, 1e-4), "ceil": (3e-5, 3e-5, 1e-4)}


def check_tanh_closed_form(rules=("ocp", "plus1", "ceil")):
    bits = workloads.tanh_activations(rows=1024, cols=4096)
    x = bulk.bf16_bits_to_f64(bits.ravel())
    for rule in rules:
        want = tanh_expected(rule)
        assert abs(want["p_total"] - 1.0) < 1e-12
        codes, sc, _ = bulk.cast_mx_f64(E4M3, x, 4096, rule)
        K = -bulk.mx_element_exponents(sc.astype(np.int64) - 127, x.size, 4096)
        st = bulk.stats_f64(E4M3, x, codes, K)
        got = dict(sign_aligned=st["sum_dir_e"] / x.size, kept=1 + st["sum_xe"] / st["sum_x2"],
                   rel_rms=math.sqrt(st["sum_e2"] / st["sum_x2"]))
        b_bias, b_kept, b_rms = TANH_BANDS[rule]
        assert abs(got["sign_aligned"] - want["sign_aligned"]) < b_bias, (rule, got, want)
        assert abs(got["kept"] - want["kept"]) < b_kept, (rule, got, want)
        assert abs(got["rel_rms"] - want["rel_rms"]) < b_rms, (rule, got, want)
        # symmetric data: the plain mean error is ~0 under every rule, unlike
        # the error along each element's sign
        assert abs(st["sum_e"] / x.size) < 5e-5 < abs(got["sign_aligned"])


def test_tanh_bias_and_kept_fraction_closed_form():
    ocp = tanh_expected("ocp")
    assert -1.4e-2 < ocp["sign_aligned"] < -1.25e-2 and ocp["kept"] < 1
    assert 1.0e-3 < tanh_expected("plus1")["sign_aligned"] < 1.35e-3
    check_tanh_closed_form()


# -- planted mistakes ----------------------------------------------------------

def _t0_terms(mut):
    def terms(x, xhat):
        e = xhat - x
        s = (x > 0) - (x < 0)
        sh = (xhat > 0) - (xhat < 0)
        t = [e, abs(e), e * e, s * e, x * e, x * x]
        if mut == "e_sign":
            t = [-v for v in t[:1]] + [abs(e), e * e, -s * e, -x * e, x * x]
        elif mut == "abs_dropped":
            t[1] = e
        elif mut == "square_of_x":
            t[2] = x * x
        elif mut == "sign_of_xhat":
            t[3] = sh * e
        elif mut == "xhat_e":
            t[4] = xhat * e
        elif mut == "xhat_squared":
            t[5] = xhat * xhat
        return tuple(t)
    return terms


def _t1_terms(mut):
    def terms(x, xh):
        e = xh - x
        t = [e, np.abs(e), e * e, np.sign(x) * e, x * e, x * x]
        if mut == "e_sign":
            t = [-e, np.abs(e), e * e, -np.sign(x) * e, -x * e, x * x]
        elif mut == "abs_dropped":
            t[1] = e
        elif mut == "square_of_x":
            t[2] = x * x
        elif mut == "sign_of_xhat":
            t[3] = np.sign(xh) * e
        elif mut == "xhat_e":
            t[4] = xh * e
        elif mut == "xhat_squared":
            t[5] = xh * xh
        return t
    return terms


def _t0_represented_up(fmt, code, K):
    v = fmt.decode(code)
    return v if v.kind != "num" else Val.num(v.neg, v.mag * Fraction(2) ** K)


def _t1_represented_up(fmt, codes, K):
    return np.ldexp(bulk.decode_table(fmt)[np.asarray(codes, dtype=np.uint8)], np.asarray(K, dtype=np.int64))


MUTANTS = ["e_sign", "abs_dropped", "square_of_x", "sign_of_xhat", "xhat_e", "xhat_squared"]


@pytest.mark.parametrize("mut", MUTANTS)
def test_pins_catch_planted_statistics_mistakes(mut, monkeypatch):
    monkeypatch.setattr(t0, "stats_terms", _t0_terms(mut))
    with pytest.raises(AssertionError):
        check_terms_tier0()
    with pytest.raises(AssertionError):
        check_sums()
    monkeypatch.undo()
    monkeypatch.setattr(bulk, "stats_terms_f64", _t1_terms(mut))
    with pytest.raises(AssertionError):
        check_terms_tier1()
    with pytest.raises(AssertionError):
        check_sums()


def test_pins_catch_a_scale_applied_the_wrong_way(monkeypatch):
    monkeypatch.setattr(t0, "represented", _t0_represented_up)
    with pytest.raises(AssertionError):
        check_dequant()
    with pytest.raises(AssertionError):
        check_terms_tier0()
    monkeypatch.undo()
    monkeypatch.setattr(bulk, "represented_f64", _t1_represented_up)
    with pytest.raises(AssertionError):
        check_dequant()
    with pytest.raises(AssertionError):
        check_terms_tier1()


def test_closed_form_catches_xhat_e_and_a_flipped_sign(monkeypatch):
    """The tanh closed form alone also separates the plausible mistakes in
    the bulk statistics (on the OCP rule, where the effects are largest)."""
    for mut in ("xhat_e", "e_sign"):
        monkeypatch.setattr(bulk, "stats_terms_f64", _t1_terms(mut))
        with pytest.raises(AssertionError):
            check_tanh_closed_form(rules=("ocp",))
        monkeypatch.undo()
