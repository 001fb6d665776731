"""Pins of the update/step-ratio monitor's oracle: the pages' own examples,
tier 0 against tier 1, the no-op decision against the format's neighbours
found independently (numpy float16 / bf16 bit patterns), and the window rule
against a closed form."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import bulk, swamp
from oracle.formats import BF16, FP16, FP32, Val

WF = [BF16, FP16]


def test_pages_examples():
    # [E3, "Worked solution"]: adding 0.001 to a bf16 weight of 1.0 leaves it unchanged
    assert swamp.element(BF16, Val.of(1.0), Val.of(0.001)) == (True, True, False, False)
    # [SP, "Master weights ..."]: weight ~1, update ~1e-7: a no-op in 16 bits, lands in 32 bits
    for f in (BF16, FP16):
        assert swamp.element(f, Val.of(1.0), Val.of(1e-7))[1] is True
    assert swamp.element(FP32, Val.of(1.0), Val.of(1e-7))[1] is False
    # fp16's step at 1.0 is 2^-10 < 0.001: the update moves the fp16 weight
    assert swamp.element(FP16, Val.of(1.0), Val.of(0.001)) == (False, False, False, False)


def _pairs(seed, n):
    r = np.random.default_rng(seed)
    w = (r.standard_normal(n) * np.exp2(r.integers(-30, 30, n))).astype(np.float32).astype(np.float64)
    rel = np.exp2(r.uniform(-40, 5, n)) * r.choice([-1.0, 1.0], n)
    d = (w * rel).astype(np.float32).astype(np.float64)
    d[r.random(n) < 0.05] = 0.0
    w[:12] = [0.0, -0.0, 1.0, -1.0, 2.0 ** -130, 3e38, np.inf, np.nan, 65504.0, 65520.0, 2.0 ** -24, 1.5]
    d[:12] = [1e-45, -1e-45, 2.0 ** -9, 2.0 ** -9, 2.0 ** -140, 1.0, 1.0, 1.0, 16.0, 1.0, -2.0 ** -25, np.inf]
    return w, d


def _ties(fmt, seed, n):
    """Weights on F's grid and updates exactly half a gap (up or down) away,
    including powers of two, where the gap below is half the gap above."""
    r = np.random.default_rng(seed)
    wf = bulk.bf16_bits_to_f64(r.integers(0, 0x7F00, n).astype(np.uint16)) if fmt is BF16 else \
        r.integers(0, 0x7BFF, n).astype(np.uint16).view(np.float16).astype(np.float64)
    wf[: n // 4] = np.exp2(r.integers(-20, 20, n // 4)).astype(np.float64)
    wf = wf[np.isfinite(wf)]
    sign = r.choice([-1.0, 1.0], wf.size)
    wf = wf * sign
    up = _next(fmt, wf, np.inf) - wf
    dn = wf - _next(fmt, wf, -np.inf)
    d = np.where(r.random(wf.size) < 0.5, up / 2, -dn / 2)
    return wf, d


def _next(fmt, v, to):
    """The neighbour of grid values v toward `to`, from the format's own bit
    patterns (numpy float16; bf16 patterns stepped by one)."""
    if fmt is FP16:
        with np.errstate(over="ignore"):
            return np.nextafter(v.astype(np.float16), np.asarray(to).astype(np.float16)).astype(np.float64)
    bits = bulk.round_bf16_bits(v).astype(np.int64)
    mag, neg = bits & 0x7FFF, (bits >> 15) & 1
    toward_up = (to > 0) == (neg == 0)
    m2 = np.where(toward_up, mag + 1, mag - 1)
    zero_cross = (mag == 0) & ~toward_up
    b2 = np.where(zero_cross, (1 - neg) << 15 | 1, neg << 15 | np.maximum(m2, 0))
    return bulk.bf16_bits_to_f64(b2.astype(np.uint16))


@pytest.mark.parametrize("fmt", WF, ids=["bf16", "fp16"])
def test_tier0_vs_tier1(fmt):
    w, d = _pairs(1, 4000)
    wt, dt = _ties(fmt, 2, 400)
    w, d = np.concatenate([w, wt]), np.concatenate([d, dt.astype(np.float32).astype(np.float64)])
    f1, c1 = swamp.watch_f64(fmt, w, d)
    f0, c0 = swamp.watch(fmt, bulk.to_vals(w), bulk.to_vals(d))
    assert f1.tolist() == f0 and c1 == c0


@pytest.mark.parametrize("fmt", WF, ids=["bf16", "fp16"])
def test_noop_against_neighbours(fmt):
    """No-op <=> |d| is below half the gap to the neighbour on d's side, or
    exactly half with w_F's last significand bit even (ties to even); below
    <=> |d| < the gap above |w_F| -- gaps from the format's own neighbours."""
    w, d = _pairs(3, 6000)
    wt, dt = _ties(fmt, 4, 2000)
    w, d = np.concatenate([w, wt]), np.concatenate([d, dt])
    flags, _ = swamp.watch_f64(fmt, w, d)
    keep = (flags & 0b1100) == 0
    w, d, flags = w[keep], d[keep], flags[keep]
    wf = swamp._round_to(fmt, w)
    top = np.abs(wf) < float(fmt.maxval)
    w, d, wf, flags = w[top], d[top], wf[top], flags[top]
    nb = _next(fmt, wf, np.where(d > 0, np.inf, -np.inf))
    half = np.abs(nb - wf) / 2
    if fmt is FP16:
        even = (wf.astype(np.float16).view(np.uint16) & 1) == 0
    else:
        even = (bulk.round_bf16_bits(wf) & 1) == 0
    want_noop = (np.abs(d) < half) | ((np.abs(d) == half) & even)
    assert np.array_equal((flags >> 1) & 1, want_noop.astype(np.uint8))
    gap_up = np.abs(_next(fmt, np.abs(wf), np.inf) - np.abs(wf))
    assert np.array_equal(flags & 1, (np.abs(d) < gap_up).astype(np.uint8))
    assert 0 < want_noop.sum() < want_noop.size


def test_window_rule_closed_form():
    """promoted after step t <=> some W consecutive steps up to t were below;
    run = the length of the trailing below streak."""
    for W in (1, 2, 3, 4):
        p = swamp.WindowPolicy(window=W, num=1, den=2)
        for seq in itertools.product([0, 1], repeat=7):
            s = swamp.WindowState()
            for t, b in enumerate(seq):
                c = dict(n_considered=10, n_below=5 if b else 4)
                s = swamp.window_step(p, s, c)
                prefix = "".join(map(str, seq[:t + 1]))
                assert s.promoted == int("1" * W in prefix)
                assert s.run == len(prefix) - len(prefix.rstrip("1"))
                assert s.steps == t + 1


def test_window_threshold_and_empty():
    p = swamp.WindowPolicy(window=1, num=3, den=4)
    s = swamp.WindowState()
    assert swamp.window_step(p, s, dict(n_considered=4, n_below=2)).promoted == 0
    assert swamp.window_step(p, s, dict(n_considered=4, n_below=3)).promoted == 1
    assert swamp.window_step(p, s, dict(n_considered=0, n_below=0)).run == 0
    big = 1 << 34
    assert swamp.window_step(p, s, dict(n_considered=big, n_below=3 * big // 4)).promoted == 1
    assert swamp.window_step(p, s, dict(n_considered=big, n_below=3 * big // 4 - 1)).promoted == 0
