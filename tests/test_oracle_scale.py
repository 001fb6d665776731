"""Pins of the scale rules (per-tensor and MX) and their invariants."""

import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.stats import norm

from oracle import E4M3, E5M2, Val
from oracle import bulk
from oracle import cast as t0
from oracle.formats import pow2
import workloads


def F(*x):
    return Fraction(*x)


# Worked by hand from the rule "largest power of two keeping amax * scale
# <= 448" (E4M3) / "<= 57344" (E5M2).
HAND = [
    (E4M3, F(1), 0, 8),            # 256 <= 448 < 512
    (E4M3, F(448), 0, 0),
    (E4M3, F(448) + pow2(-15), 0, -1),
    (E4M3, F(9, 2), 0, 6),         # 4.5 * 64 = 288; * 128 = 576
    (E4M3, F(7, 2), 0, 7),         # 3.5 * 128 = 448 exactly
    (E4M3, F(7, 2) + pow2(-22), 0, 6),
    (E4M3, F(1), 1, 7),            # margin of one binade: bound 224
    (E4M3, F(0), 0, 127),
    (E4M3, pow2(-149), 0, 127),    # would be 157: clamped
    (E4M3, pow2(127), 0, -119),
    (E5M2, F(1), 0, 15),           # 32768 <= 57344 < 65536
    (E5M2, F(57344), 0, 0),
    (E5M2, F(7, 4) * pow2(-20), 0, 35),
]


@pytest.mark.parametrize("fmt,a,margin,k", HAND)
def test_scale_exponent_hand_values(fmt, a, margin, k):
    assert t0.scale_exponent(fmt, a, margin) == k


def test_scale_exponent_is_largest():
    """For many estimates: a * 2^k fits and a * 2^(k+1) does not (unless k is
    at the clamp)."""
    rng = np.random.default_rng(0)
    for fmt in (E4M3, E5M2):
        for _ in range(2000):
            a = Fraction(float(np.float32(np.exp2(rng.uniform(-140, 127)))))
            m = int(rng.integers(0, 3))
            k = t0.scale_exponent(fmt, a, m)
            bound = fmt.maxval * pow2(-m)
            assert k == 127 or a * pow2(k + 1) > bound
            assert k == -127 or a * pow2(k) <= bound


def test_current_scaling_never_clips():
    """[E3, "Worked solution"]: the run did not overflow, by construction.
    Under current scaling (scale from this tensor's own amax) no element
    clips, on any data."""
    for seed in range(6):
        x = workloads.mixed_magnitude_fp32(5000, seed, -60 + 10 * seed, 10 * seed).astype(np.float64)
        for fmt in (E4M3, E5M2):
            k = t0.scale_exponent(fmt, Fraction(bulk.amax_f64(x)))
            codes, counts = bulk.cast_tensor_f64(fmt, x, k)
            assert counts["n_clip"] == 0


def test_per_tensor_small_workload_expectations():
    """65,536 N(0, 1) samples: amax between 4 and 7 gives k = 6 (scale 64);
    no clips; underflows are |x| <= 2^-16, about 0.8 expected."""
    x = workloads.per_tensor_small().astype(np.float64)
    a = bulk.amax_f64(x)
    assert 4 <= a < 7
    k = t0.scale_exponent(E4M3, Fraction(a))
    assert k == 6
    codes, counts = bulk.cast_tensor_f64(E4M3, x, k)
    assert counts["n_clip"] == 0
    assert counts["n_underflow"] == int(np.count_nonzero((np.abs(x) <= 2.0 ** -16) & (x != 0)))
    assert counts["n_underflow"] <= 5


# -- MX rules -------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [E4M3, E5M2], ids=["e4m3", "e5m2"])
def test_mx_rule_closed_forms(fmt):
    """OCP: an element clips exactly when |x| > 1.75 * 2^e(block amax);
    +1 headroom and round-up never clip."""
    rng = np.random.default_rng(4)
    x = (np.tanh(rng.normal(0, 1.5, 64 * 32)) * np.repeat(np.exp2(rng.integers(-20, 20, 64)), 32))
    x = x.astype(np.float32).astype(np.float64)
    for rule in ("ocp", "plus1", "ceil"):
        codes, scales, counts = bulk.cast_mx_f64(fmt, x, 32, rule)
        if rule == "ocp":
            blocks = x.reshape(-1, 32)
            a = np.abs(blocks).max(axis=1)
            thr = 1.75 * np.exp2(np.floor(np.log2(a)))
            assert counts["n_clip"] == int(np.count_nonzero(np.abs(blocks) > thr[:, None]))
            assert counts["n_clip"] > 0
        else:
            assert counts["n_clip"] == 0
    for a in (F(1), F(7, 8), F(15, 16), F(1, 3), pow2(-140), F(57344)):
        ocp = t0.mx_exponent(fmt, a, "ocp")
        assert a * pow2(-ocp) >= pow2(fmt.emax) and a * pow2(-ocp) < pow2(fmt.emax + 1) or ocp == -127
        raw = math.floor(math.log2(a)) - fmt.emax
        assert ocp == max(-127, raw)
        assert t0.mx_exponent(fmt, a, "plus1") == max(-127, min(127, raw + 1))
        c = t0.mx_exponent(fmt, a, "ceil")
        assert a * pow2(-c) <= fmt.maxval and (a * pow2(-(c - 1)) > fmt.maxval or c == -127)


def test_tanh_workload_clip_fraction_closed_form():
    """bf16 tanh(N(0, 1.5)) under the OCP rule.  A block whose largest
    element rounded to exactly 1.0 in bf16 never clips; otherwise (block amax
    in [0.5, 1)) an element clips when its bf16 value exceeds 0.875, i.e. its
    magnitude exceeds 0.875 + 2^-9.  Expected fraction
    (P(|t| > 0.875 + 2^-9) - p1) (1 - p1)^31 with p1 = P(|t| >= 1 - 2^-9).
    The +1 rule never clips.  (The pages' 27-30% came from trained models'
    activations; this synthetic stand-in differs, as derived here.)"""
    sd = 1.5

    def p_abs_tanh_above(c):
        return 2 * norm.sf(math.atanh(c) / sd)

    p1 = p_abs_tanh_above(1 - 2.0 ** -9)
    expected = (p_abs_tanh_above(0.875 + 2.0 ** -9) - p1) * (1 - p1) ** 31
    assert 0.17 < expected < 0.19
    bits = workloads.tanh_activations(rows=1024, cols=4096)
    x = bulk.bf16_bits_to_f64(bits.ravel())
    _, _, c_ocp = bulk.cast_mx_f64(E4M3, x, 4096, "ocp")
    _, _, c_p1 = bulk.cast_mx_f64(E4M3, x, 4096, "plus1")
    frac = c_ocp["n_clip"] / x.size
    assert abs(frac - expected) < 0.003, (frac, expected)
    assert c_p1["n_clip"] == 0


def test_unscale_identity():
    """A power-of-two loss scale makes the unscale exact, so unscale-then-cast
    at k equals a cast at k - s, bit for bit, for normal fp32 inputs."""
    x = workloads.mixed_magnitude_fp32(3000, 21, -100, 100).astype(np.float64)
    for s in (0, 16, 24):
        xu = np.ldexp(x, -s)
        for k in (3, -5, 40):
            a = bulk.cast_f64(E4M3, xu, k)
            b = bulk.cast_f64(E4M3, x, k - s)
            for u, v in zip(a, b):
                assert np.array_equal(u, v)


def test_tier0_cast_tensor_counts():
    vals = [Val.of(v) for v in (1.0, -500.0, 2.0 ** -12, math.inf, math.nan, -0.0)]
    codes, counts = t0.cast_tensor(E4M3, vals, 0)
    assert codes == [0x38, 0xFE, 0x00, 0x7E, 0x7F, 0x80]
    assert counts == dict(n_finite=4, n_clip=1, n_underflow=1, n_nonfinite=2, amax=Fraction(500))
